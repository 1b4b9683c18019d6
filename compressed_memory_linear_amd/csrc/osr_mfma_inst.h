// osr_mfma_inst.h -- launch of the MFMA chunk kernels for one slot count M
// (included once per M by osr_mfma_m*.hip so the instantiations compile in
// parallel).
#pragma once

#include "osr_launch.h"
#include "osr_mfma_kernels.h"
#include "osr_mfma_readout.h"

namespace osr {
namespace mfma {

// Sub-block length C0 (<= C) of the fused kernel.  Longer sub-blocks mean
// fewer barriers per chunk but more live registers (gates, H fragments and
// the prefetched inputs grow with C0); it stays at <= 32 because its causal
// block grows as C0^2, and at 16 for d = 128 to stay within the register file.
template <int M, int D, bool WITH_Y>
constexpr bool fits_c0(int c0) {
    return c0 == 64 ? fits<M, D, 64, WITH_Y>() : c0 == 32 ? fits<M, D, 32, WITH_Y>() : fits<M, D, 16, WITH_Y>();
}
// Sub-block of the split schedule's read-out kernel: 32 tokens (the running
// gate products stay within a short window), 16 where C is 16 and for
// m = 128 with one wave (d = 16), which would spill at 32.
template <int M, int D>
constexpr int pick_c0_split_readout(int C) {
    return C >= 32 && readout_fits<M, D, 32>() && !(M == 128 && D == 16) ? 32 : 16;
}
template <int M, int D>
constexpr int pick_c0_fused(int C) {
    int c0 = D == 128 ? 16 : 32;
    while (c0 > 16 && (c0 > C || !fits_c0<M, D, true>(c0))) c0 /= 2;
    return c0;
}
// State-passing kernel, instantiated in osr_chain_m*.hip (built with MFMA
// results in VGPRs).
template <int M>
int launch_chain_m(int d, const Params& p, hipStream_t st);

template <int M, int D, int C0>
static int launch_fused(const Params& p, hipStream_t st) {
    if constexpr (!fits<M, D, C0, true>()) {
        return -3;
    } else {
        const unsigned BH = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H);
        hipLaunchKernelGGL((osr_fused_kernel<M, D, C0>), dim3(BH), dim3(4 * D), 0, st, p);
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D, int C0>
static int launch_readout(const Params& p, hipStream_t st) {
    if constexpr (!readout_fits<M, D, C0>() || !readout_fits<M, D, C0, true>()) {
        // (every built m, d and sub-block fits both layouts)
        return -3;
    } else {
        // the launch's chunk range
        const int BH = p.B * p.H, NC = (p.n_end > 0 ? p.n_end : p.T / p.chunk) - p.n_begin;
        // At least 512 workgroups (the kernel's registers and LDS hold two per
        // CU); each takes cpw consecutive chunks (a power of two dividing NC),
        // which keeps the register prefetch running across chunk boundaries.
        int cpw = 1;
        while (cpw * 2 <= NC && NC % (cpw * 2) == 0 && static_cast<int64_t>(BH) * NC / (cpw * 2) >= 512) cpw *= 2;
        const unsigned grid = static_cast<unsigned>(BH) * static_cast<unsigned>(NC / cpw);
        if (p.lin1)
            hipLaunchKernelGGL((osr_readout_kernel<M, D, C0, true>), dim3(grid), dim3(4 * D), 0, st, p, cpw);
        else
            hipLaunchKernelGGL((osr_readout_kernel<M, D, C0, false>), dim3(grid), dim3(4 * D), 0, st, p, cpw);
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D>
static int launch_readout_md(const Params& p, hipStream_t st) {
    return pick_c0_split_readout<M, D>(p.chunk) == 32 ? launch_readout<M, D, 32>(p, st)
                                                      : launch_readout<M, D, 16>(p, st);
}

// Split schedule with the read-out overlapped (ov set): the chunks in ov->nseg
// ranges; range k's state passing runs on the caller's stream st, and its
// read-out on the side stream once that range's state passing is done, while
// range k + 1's state passing runs; the last read-out runs on st, which then
// waits for the side stream.  The ranges hand the state on through p.carry.
template <int M, int D>
static int launch_md(bool split, const Params& p, hipStream_t st, const Overlap* ov) {
    const int C = p.chunk;
    const int c0 = pick_c0_fused<M, D>(C);
    if (split) {
        if (!ov) {
            const int rc = launch_chain_m<M>(D, p, st);
            if (rc) return rc;
            return launch_readout_md<M, D>(p, st);
        }
        Params q = p;
        int rc = 0;
        for (int k = 0; k < ov->nseg && rc == 0; ++k) {
            q.n_begin = k == 0 ? 0 : ov->end[k - 1];
            q.n_end = ov->end[k];
            rc = launch_chain_m<M>(D, q, st);
            if (rc) break;
            if (k + 1 < ov->nseg) {
                if (hipEventRecord(ov->ev_chain, st) != hipSuccess ||
                    hipStreamWaitEvent(ov->side, ov->ev_chain, 0) != hipSuccess) {
                    rc = -5;
                    break;
                }
                rc = launch_readout_md<M, D>(q, ov->side);
            } else {
                rc = launch_readout_md<M, D>(q, st);
            }
        }
        // the caller's stream waits for whatever reached the side stream, on
        // failure too (the caller may reuse the workspace once its stream is done)
        if (hipEventRecord(ov->ev_side, ov->side) != hipSuccess ||
            hipStreamWaitEvent(st, ov->ev_side, 0) != hipSuccess)
            rc = rc ? rc : -5;
        return rc;
    }
    return c0 == 32 ? launch_fused<M, D, 32>(p, st) : launch_fused<M, D, 16>(p, st);
}

template <int M>
int launch_m(int d, bool split, const Params& p, hipStream_t st, const Overlap* ov) {
    switch (d) {
        case 16: return launch_md<M, 16>(split, p, st, ov);
        case 32: return launch_md<M, 32>(split, p, st, ov);
        case 64: return launch_md<M, 64>(split, p, st, ov);
        case 128: return launch_md<M, 128>(split, p, st, ov);
        default: return -3;
    }
}

}  // namespace mfma
}  // namespace osr
