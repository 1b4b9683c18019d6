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

// Workgroups per sequence of the small-chunk walk: 2 (half the slot rows each,
// half the VALU issue per chunk, one hand-off per chunk) where each keeps at
// least 16 rows, the chunk has at least 4 tokens and B*H*2 <= 256 (one
// workgroup per compute unit, all resident: they wait for each other);
// chain_wgs != 0 asks for one.  The hand-off (stores retired, counter, poll,
// loads) costs ~6.5k cycles per chunk: B4 H8 T2048 m = d = 64 measured 5.87
// against 5.40 ms at C = 2, 4.39 against 4.57 at C = 4, 3.69 against 4.19 at
// C = 8.
int bwd_small_split_p(int B, int H, int m, int C, int chain_wgs) {
    if (chain_wgs != 0 || m / 2 < 16 || C < 4) return 1;
    return static_cast<int64_t>(B) * H * 2 <= 256 ? 2 : 1;
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
