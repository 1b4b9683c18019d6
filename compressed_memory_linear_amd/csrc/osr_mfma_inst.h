// osr_mfma_inst.h -- launch of the MFMA chunk kernels for one slot count M
// (included once per M by osr_mfma_m*.hip so the instantiations compile in
// parallel).
#pragma once

#include "osr_launch.h"
#include "osr_mfma_chain.h"
#include "osr_mfma_kernels.h"

namespace osr {
namespace mfma {

// Sub-block length C0 (<= C) of the read-out kernels.  Longer sub-blocks
// mean fewer barriers per chunk but more live registers (gates, H fragments
// and the prefetched inputs grow with C0); the read-out kernels stay at <= 32
// because their causal block grows as C0^2, and at 16 for d = 128 to stay
// within the register file.
template <int M, int D, bool WITH_Y>
constexpr bool fits_c0(int c0) {
    return c0 == 64 ? fits<M, D, 64, WITH_Y>() : c0 == 32 ? fits<M, D, 32, WITH_Y>() : fits<M, D, 16, WITH_Y>();
}
template <int M, int D>
constexpr int pick_c0_readout(int C) {
    int c0 = D == 128 ? 16 : 32;
    while (c0 > 16 && (c0 > C || !fits_c0<M, D, true>(c0))) c0 /= 2;
    return c0;
}
// The state-passing kernel takes whole chunks where LDS and the register
// file allow (one sub-block per chunk: two barriers per chunk); 64-token
// sub-blocks spill when one lane row holds d = 128 columns of state with
// fewer than 4 waves, or with 8 waves (2 per SIMD) from d = 64 up.
template <int M, int D>
constexpr bool chain_fits_c0(int c0) {
    return c0 == 64 ? chain_fits<M, D, 64>() : c0 == 32 ? chain_fits<M, D, 32>() : chain_fits<M, D, 16>();
}
template <int M, int D>
constexpr int pick_c0_chain(int C) {
    int c0 = (D == 128 && M <= 64) || (M == 128 && D >= 64) ? 32 : 64;
    while (c0 > 16 && (c0 > C || !chain_fits_c0<M, D>(c0))) c0 /= 2;
    return c0;
}

template <int M, int D, int C0>
static int launch_chain(const Params& p, hipStream_t st) {
    if constexpr (!chain_fits<M, D, C0>()) {
        return -3;
    } else {
        const unsigned BH = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H);
        hipLaunchKernelGGL((osr_chain_kernel<M, D, C0, true>), dim3(BH), dim3(4 * M), 0, st, p);
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D, int C0, bool WITH_Y, bool WRITE_Z>
static int launch_loop(const Params& p, hipStream_t st) {
    if constexpr (!fits<M, D, C0, WITH_Y>()) {
        return -3;
    } else {
        const unsigned BH = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H);
        hipLaunchKernelGGL((osr_chunk_loop_kernel<M, D, C0, WITH_Y, WRITE_Z>), dim3(BH), dim3(4 * D), 0, st, p);
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D, int C0>
static int launch_intra(const Params& p, hipStream_t st) {
    if constexpr (!fits<M, D, C0, true>()) {
        return -3;
    } else {
        const int BH = p.B * p.H, NC = p.T / p.chunk;
        // Enough workgroups for every CU at the occupancy LDS allows; each
        // takes cpw consecutive chunks (a power of two dividing NC).
        const int per_cu = (160 * 1024) / Cfg<M, D, C0, true>::BYTES;
        const int64_t target = 256LL * (per_cu > 0 ? per_cu : 1);
        int cpw = 1;
        while (cpw * 2 <= NC && NC % (cpw * 2) == 0 && static_cast<int64_t>(BH) * NC / (cpw * 2) >= target) cpw *= 2;
        const unsigned grid = static_cast<unsigned>(BH) * static_cast<unsigned>(NC / cpw);
        hipLaunchKernelGGL((osr_intra_chunk_kernel<M, D, C0>), dim3(grid), dim3(4 * D), 0, st, p, cpw);
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D>
static int launch_md(bool split, const Params& p, hipStream_t st) {
    const int C = p.chunk;
    const int c0 = pick_c0_readout<M, D>(C);
    if (split) {
        int rc;
        switch (pick_c0_chain<M, D>(C)) {
            case 64: rc = launch_chain<M, D, 64>(p, st); break;
            case 32: rc = launch_chain<M, D, 32>(p, st); break;
            default: rc = launch_chain<M, D, 16>(p, st); break;
        }
        if (rc) return rc;
        return c0 == 32 ? launch_intra<M, D, 32>(p, st) : launch_intra<M, D, 16>(p, st);
    }
    return c0 == 32 ? launch_loop<M, D, 32, true, false>(p, st) : launch_loop<M, D, 16, true, false>(p, st);
}

template <int M>
int launch_m(int d, bool split, const Params& p, hipStream_t st) {
    switch (d) {
        case 16: return launch_md<M, 16>(split, p, st);
        case 32: return launch_md<M, 32>(split, p, st);
        case 64: return launch_md<M, 64>(split, p, st);
        case 128: return launch_md<M, 128>(split, p, st);
        default: return -3;
    }
}

}  // namespace mfma
}  // namespace osr
