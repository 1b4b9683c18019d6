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

template <int M, int D, int C0>
static int launch_chain(const Params& p, hipStream_t st) {
    if constexpr (!chain_fits<M, D, C0>()) {
        return -3;
    } else {
        const unsigned BH = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H);
        if (p.chunk == C0)
            hipLaunchKernelGGL((osr_chain_kernel<M, D, C0, true, true>), dim3(BH), dim3(4 * M), 0, st, p);
        else
            hipLaunchKernelGGL((osr_chain_kernel<M, D, C0, true, false>), dim3(BH), dim3(4 * M), 0, st, p);
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D>
static int launch_chain_md(const Params& p, hipStream_t st) {
    switch (pick_c0_chain<M, D>(p.chunk)) {
        case 64: return launch_chain<M, D, 64>(p, st);
        case 32: return launch_chain<M, D, 32>(p, st);
        default: return launch_chain<M, D, 16>(p, st);
    }
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
