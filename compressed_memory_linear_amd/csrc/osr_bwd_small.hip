// osr_bwd_small.hip -- dispatch of the small-chunk reverse walk (kernels:
// osr_bwd_small.h, instantiated per slot count in osr_bwd_small_m<M>.hip).
#include "osr_bwd_small.h"

namespace osr {

template <int M>
int launch_bwd_small_m(int d, const BwdParams& p, bool in_bf16, hipStream_t st);
extern template int launch_bwd_small_m<16>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_small_m<32>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_small_m<64>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_small_m<128>(int, const BwdParams&, bool, hipStream_t);

bool bwd_small_supported(int m, int d, int C, bool lin1) {
    if (lin1) return false;
    switch (m) {
        case 16: return bwd_small_fits_m<16>(d, C);
        case 32: return bwd_small_fits_m<32>(d, C);
        case 64: return bwd_small_fits_m<64>(d, C);
        case 128: return bwd_small_fits_m<128>(d, C);
        default: return false;
    }
}

int launch_bwd_small(int m, int d, const BwdParams& p, bool in_bf16, hipStream_t st) {
    switch (m) {
        case 16: return launch_bwd_small_m<16>(d, p, in_bf16, st);
        case 32: return launch_bwd_small_m<32>(d, p, in_bf16, st);
        case 64: return launch_bwd_small_m<64>(d, p, in_bf16, st);
        case 128: return launch_bwd_small_m<128>(d, p, in_bf16, st);
        default: return -3;
    }
}

}  // namespace osr
