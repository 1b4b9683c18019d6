// osr_mfma_inst.h -- launch of the MFMA chunk kernels for one slot count M
// (included once per M by osr_mfma_m*.hip so the instantiations compile in
// parallel).
#pragma once

#include "osr_launch.h"
#include "osr_mfma_kernels.h"

namespace osr {
namespace mfma {

template <int M, int D, int C0>
static int launch_mdc(bool split, const Params& p, hipStream_t st) {
    if constexpr (!fits<M, D, C0>()) {
        return -3;
    } else {
        using G = Cfg<M, D, C0>;
        const unsigned BH = static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H);
        if (split) {
            const unsigned NC = static_cast<unsigned>(p.T / p.chunk);
            hipLaunchKernelGGL((osr_chunk_loop_kernel<M, D, C0, false, true>), dim3(BH), dim3(G::NT), 0, st, p);
            if (hipGetLastError() != hipSuccess) return -5;
            hipLaunchKernelGGL((osr_intra_chunk_kernel<M, D, C0>), dim3(BH * NC), dim3(G::NT), 0, st, p);
        } else {
            hipLaunchKernelGGL((osr_chunk_loop_kernel<M, D, C0, true, false>), dim3(BH), dim3(G::NT), 0, st, p);
        }
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D>
static int launch_md(int c0, bool split, const Params& p, hipStream_t st) {
    return c0 == 32 ? launch_mdc<M, D, 32>(split, p, st) : launch_mdc<M, D, 16>(split, p, st);
}

template <int M>
int launch_m(int d, int c0, bool split, const Params& p, hipStream_t st) {
    switch (d) {
        case 16: return launch_md<M, 16>(c0, split, p, st);
        case 32: return launch_md<M, 32>(c0, split, p, st);
        case 64: return launch_md<M, 64>(c0, split, p, st);
        case 128: return launch_md<M, 128>(c0, split, p, st);
        default: return -3;
    }
}

}  // namespace mfma
}  // namespace osr
