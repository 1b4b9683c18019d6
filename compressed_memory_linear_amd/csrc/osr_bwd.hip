// osr_bwd.hip -- dispatch and workspace size of the backward of the chunk-wise
// OSR forward (kernels: osr_bwd_kernel.h, instantiated per slot count in
// osr_bwd_m<M>.hip).
#include "osr_launch.h"

namespace osr {

template <int M>
int launch_bwd_m(int d, const BwdParams& p, bool in_bf16, hipStream_t st);
extern template int launch_bwd_m<16>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_m<32>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_m<64>(int, const BwdParams&, bool, hipStream_t);
extern template int launch_bwd_m<128>(int, const BwdParams&, bool, hipStream_t);

int launch_bwd(int m, int d, const BwdParams& p, bool in_bf16, hipStream_t st) {
    switch (m) {
        case 16: return launch_bwd_m<16>(d, p, in_bf16, st);
        case 32: return launch_bwd_m<32>(d, p, in_bf16, st);
        case 64: return launch_bwd_m<64>(d, p, in_bf16, st);
        case 128: return launch_bwd_m<128>(d, p, in_bf16, st);
        default: return -3;
    }
}

// Workspace floats per (b,h): the T/C + 1 chunk-start states, the running state
// before each token of one chunk, and per token c, beta (m each), |h|^2 and pad.
static size_t bwd_floats(int T, int m, int d, int C) {
    return (static_cast<size_t>(T / C) + 1 + C) * m * d + static_cast<size_t>(C) * (2 * m + 4);
}

size_t bwd_workspace_bytes(int B, int H, int T, int m, int d, int C) {
    return bwd_floats(T, m, d, C) * sizeof(float) * static_cast<size_t>(B) * static_cast<size_t>(H);
}

// The reverse walk's per-token work is per slot row except the sums over slots
// of each batch of tokens, so the rows of one sequence split over P workgroups
// that exchange those sums.  Where the state-passing kernel supplies the
// chunk-start states and records (bf16 inputs, C >= 16, decoding and similarity
// objectives): the largest P in {1, 2, 4, 8} with at least 16 rows per
// workgroup, B*H*P <= 256 (one workgroup per compute unit, all resident) and
// the workgroup's LDS (exchange buffers, the chunk's h and, at <= 32 rows and
// <= 2 per thread, its rows' records and, at d <= 64, the chunk's dy; the
// kernel's layout) within 160 KiB.
bool bwd_split_fits(int m, int d, int C, int P) {
    const int ML = m / P, TPR = d / 4, NT = ML * TPR < 512 ? ML * TPR : 512, RG = NT / TPR, RPT = ML / RG;
    const int NW = NT / 64, W = d + 4;
    const bool stg = P > 1 && RPT <= 2 && ML <= 32;
    // (the kernel's WalkBatch: the chunk's h batch BTC, the walk's batch BT)
    int BTC = RPT <= 2 ? 8 : (RPT <= 4 ? 4 : 2);
    if (TPR == 32 && BTC > 4) BTC = 4;
    const int BT = stg && TPR == 32 && BTC < 8 ? 8 : BTC;
    const size_t red = static_cast<size_t>(2 * BTC > BT ? 2 * BTC : BT) * NW * W;
    size_t lds = (red + static_cast<size_t>(BT) * W) * 4 + static_cast<size_t>(C) * d * 4;
    if (stg) lds += ((5 * static_cast<size_t>(ML) + 3) * C + (d <= 64 ? static_cast<size_t>(C) * d : 0)) * 4;
    return lds <= 160 * 1024;
}

int bwd_split_p(int B, int H, int m, int d, int C, bool chain, int chain_wgs) {
    if (!chain || chain_wgs != 0) return 1;
    const int64_t bh = static_cast<int64_t>(B) * H;
    int best = 1;
    for (int P = 2; P <= 8 && m / P >= 16 && bh * P <= 256; P *= 2)
        if (bwd_split_fits(m, d, C, P)) best = P;
    return best;
}

// Per (b,h): 2 parities x P parts of at most 8 tokens x (d + 4) floats, then P
// counters of XFLAG_STRIDE ints.
size_t bwd_xchg_bytes(int B, int H, int d, int P) {
    if (P <= 1) return 0;
    const size_t bh = static_cast<size_t>(B) * H;
    return bh * (2 * static_cast<size_t>(P) * 8 * (d + 4) * sizeof(float) + static_cast<size_t>(P) * XFLAG_STRIDE * sizeof(int));
}

}  // namespace osr
