// osr_chain_inst.h -- launch of the state-passing kernel for one slot count M
// (included once per M by osr_chain_m*.hip).
#pragma once

#include "osr_launch.h"
#include "osr_mfma_chain.h"

namespace osr {
namespace mfma {

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

// Two waves per slot block (two token halves per chunk) when a chunk is one
// sub-block of at least two token tiles and m <= 32: there the one-wave form
// leaves SIMDs idle (m/16 < 4 waves), and the pair form measured 10-20%
// faster (m=32 d=32 C=64: 87 vs 97 us; m=16 d=64: 129 vs 161 us for
// B4 H8 T2048).  From m = 64 every SIMD already holds one wave, the phases are
// bound by the CU's shared LDS and issue throughput, and the extra exchange
// made it slower (169 vs 159 us at m=d=64 C=64).  Params::chain_pairs = 1
// turns it off.
template <int M, int D, int C0>
constexpr bool pair_capable() {
    if constexpr (M <= 32 && C0 >= 32)
        return chain_fits<M, D, C0, true>();
    else
        return false;
}

// Sub-block length of the state-passing kernel for (d, C) at this M.
template <int M>
int chain_subblock_m(int d, int C) {
    switch (d) {
        case 16: return pick_c0_chain<M, 16>(C);
        case 32: return pick_c0_chain<M, 32>(C);
        case 64: return pick_c0_chain<M, 64>(C);
        case 128: return pick_c0_chain<M, 128>(C);
        default: return 0;
    }
}

template <int N>
__global__ void osr_zero_ints(int* x, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) x[i] = N;
}

template <int M, int D, int C0, bool ENC, bool LIN1, bool RAW>
static void launch_chain_mode(const Params& p, hipStream_t st) {
    const unsigned BH = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H);
    if constexpr (!RAW && C0 <= 64) {
        // Split over P = C / C0 workgroups per sequence (the caller set up the
        // hand-off buffers only where that applies): counters to zero first.
        if (p.xbuf && (p.chain_p == 2 || p.chain_p == 4) && p.chunk == p.chain_p * C0) {
            const int P = p.chain_p;
            const int nflags = static_cast<int>(BH) * P * (M / 16) * XFLAG_STRIDE;
            // (the counters run on across the chunk ranges of one forward: zeroed before its first)
            if (p.n_begin == 0)
                hipLaunchKernelGGL(osr_zero_ints<0>, dim3((nflags + 255) / 256), dim3(256), 0, st, p.xflags, nflags);
            const unsigned grid = (BH + 7) / 8 * 8 * static_cast<unsigned>(P);
            if (P == 2)
                hipLaunchKernelGGL((osr_chain_kernel<M, D, C0, true, false, false, ENC, LIN1, false, 2>), dim3(grid),
                                   dim3(4 * M), 0, st, p);
            else
                hipLaunchKernelGGL((osr_chain_kernel<M, D, C0, true, false, false, ENC, LIN1, false, 4>), dim3(grid),
                                   dim3(4 * M), 0, st, p);
            return;
        }
    }
    if (p.chunk != C0) {
        hipLaunchKernelGGL((osr_chain_kernel<M, D, C0, true, false, false, ENC, LIN1, RAW>), dim3(BH), dim3(4 * M), 0,
                           st, p);
        return;
    }
    if constexpr (pair_capable<M, D, C0>()) {
        if (p.chain_pairs == 0) {
            hipLaunchKernelGGL((osr_chain_kernel<M, D, C0, true, true, true, ENC, LIN1, RAW>), dim3(BH), dim3(8 * M), 0,
                               st, p);
            return;
        }
    }
    hipLaunchKernelGGL((osr_chain_kernel<M, D, C0, true, true, false, ENC, LIN1, RAW>), dim3(BH), dim3(4 * M), 0, st,
                       p);
}

template <int M, int D, int C0>
static int launch_chain(const Params& p, hipStream_t st) {
    if constexpr (!chain_fits<M, D, C0>()) {
        return -3;
    } else {
        // the encoding layer and the first linearisation are instantiations of their own
        // (the backward's raw outputs are built for the decoding and similarity objectives)
        if (p.mode == 2) {
            if (p.raw) return -3;
            if (p.lin1)
                launch_chain_mode<M, D, C0, true, true, false>(p, st);
            else
                launch_chain_mode<M, D, C0, true, false, false>(p, st);
        } else if (p.raw) {
            if (p.lin1)
                launch_chain_mode<M, D, C0, false, true, true>(p, st);
            else
                launch_chain_mode<M, D, C0, false, false, true>(p, st);
        } else {
            if (p.lin1)
                launch_chain_mode<M, D, C0, false, true, false>(p, st);
            else
                launch_chain_mode<M, D, C0, false, false, false>(p, st);
        }
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D>
static int launch_chain_md(const Params& p, hipStream_t st) {
    // Only sub-block lengths the pick can return are instantiated.
    constexpr int cmax = pick_c0_chain<M, D>(64);
    const int c0 = p.chain_p > 1 ? p.chunk / p.chain_p : pick_c0_chain<M, D>(p.chunk);
    if constexpr (cmax >= 64)
        if (c0 == 64) return launch_chain<M, D, 64>(p, st);
    if constexpr (cmax >= 32)
        if (c0 == 32) return launch_chain<M, D, 32>(p, st);
    return launch_chain<M, D, 16>(p, st);
}

template <int M>
int launch_chain_m(int d, const Params& p, hipStream_t st) {
    switch (d) {
        case 16: return launch_chain_md<M, 16>(p, st);
        case 32: return launch_chain_md<M, 32>(p, st);
        case 64: return launch_chain_md<M, 64>(p, st);
        case 128: return launch_chain_md<M, 128>(p, st);
        default: return -3;
    }
}

}  // namespace mfma
}  // namespace osr
