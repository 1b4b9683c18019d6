// osr_bwd_small.hip -- dispatch of the small-chunk reverse walk (kernels:
// osr_bwd_small.h, instantiated per slot count in osr_bwd_small_m<M>.hip).
#include "osr_bwd_small.h"

namespace osr {

// (one translation unit per (m, d): osr_bwd_small_m<M>_d<D>.hip)
#define OSR_SMALL_EXTERN(M, D) extern template int launch_bwd_small_md<M, D>(const BwdParams&, bool, hipStream_t);
#define OSR_SMALL_EXTERN_M(M) OSR_SMALL_EXTERN(M, 16) OSR_SMALL_EXTERN(M, 32) OSR_SMALL_EXTERN(M, 64) OSR_SMALL_EXTERN(M, 128)
OSR_SMALL_EXTERN_M(16)
OSR_SMALL_EXTERN_M(32)
OSR_SMALL_EXTERN_M(64)
OSR_SMALL_EXTERN_M(128)
#undef OSR_SMALL_EXTERN_M
#undef OSR_SMALL_EXTERN

template <int M>
static int launch_bwd_small_m(int d, const BwdParams& p, bool in_bf16, hipStream_t st) {
    switch (d) {
        case 16: return launch_bwd_small_md<M, 16>(p, in_bf16, st);
        case 32: return launch_bwd_small_md<M, 32>(p, in_bf16, st);
        case 64: return launch_bwd_small_md<M, 64>(p, in_bf16, st);
        case 128: return launch_bwd_small_md<M, 128>(p, in_bf16, st);
        default: return -3;
    }
}

bool bwd_small_supported(int m, int d, int C, bool lin1) {
    if (lin1 && C > 8) return false;  // (the first linearisation after the token loop only)
    switch (m) {
        case 16: return bwd_small_fits_m<16>(d, C);
        case 32: return bwd_small_fits_m<32>(d, C);
        case 64: return bwd_small_fits_m<64>(d, C);
        case 128: return bwd_small_fits_m<128>(d, C);
        default: return false;
    }
}

static bool split_ok(int m, int d, int C, int P) {
    switch (m) {
        case 16: return bwd_small_split_ok_m<16>(d, C, P);
        case 32: return bwd_small_split_ok_m<32>(d, C, P);
        case 64: return bwd_small_split_ok_m<64>(d, C, P);
        case 128: return bwd_small_split_ok_m<128>(d, C, P);
        default: return false;
    }
}

// Fewest workgroups per sequence the walk runs on at (m, d, C): 1 where a
// workgroup of the token loop's layout holds at most 2 slot rows per thread
// (m d <= 4096), else 2 or 4 (m d = 8192 at C <= 4; m = d = 128 at C = 2); 0
// where the form is not built.
int bwd_small_min_p(int m, int d, int C) {
    for (int P = 1; P <= 4; P *= 2)
        if (split_ok(m, d, C, P)) return P;
    return 0;
}

// Workgroups per sequence of the small-chunk walk (the slot rows split between
// them: fewer instructions per chunk each, one hand-off per chunk), where each
// keeps at least 16 rows and the threads to stage a chunk, and B*H*P <= 256 (one
// workgroup per compute unit, all resident: they wait for each other): 4 at
// C = 8, 2 at C = 4 (or at C = 8 where 4 do not fit), else the fewest the
// shape allows (chain_wgs != 0 asks for those).  The hand-off (~2 us per chunk)
// against the halved compute, B4 H8 T2048 m = d = 64 (ms, P = 1 / 2 / 4):
// C = 2 5.27 / 5.87 (an earlier form of the hand-off) / -, C = 4 4.61 / 4.17 /
// 4.15, C = 8 4.31 / 3.56 / 3.35.
int bwd_small_split_p(int B, int H, int m, int d, int C, int chain_wgs) {
    const int pmin = bwd_small_min_p(m, d, C);
    if (pmin == 0) return 1;
    const int64_t bh = static_cast<int64_t>(B) * H;
    int P = pmin;
    if (chain_wgs == 0) {
        if (C >= 8 && bh * 4 <= 256 && split_ok(m, d, C, 4))
            P = 4;
        else if (C >= 4 && bh * 2 <= 256 && split_ok(m, d, C, 2))
            P = P > 2 ? P : 2;
    }
    return P;
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
