// osr_launch.h -- host-side launchers of the OSR kernels (internal to the
// library; the public interface is include/lattice_osr.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

#include "osr_device.h"

namespace osr {

// VALU kernels.  decode: one exact step per (b,h) (T must be 1).
// Otherwise the token-by-token forward with chunk size p.chunk (1 = exact).
// Returns 0, -3 (unsupported m/d) or -5 (launch error).
int launch_valu(bool decode, int m, int d, const Params& p, bool in_bf16, hipStream_t st);
// The small-chunk token loop alone, at C in {1, 2, 4, 8} within its read-out
// batch (the backward's phase 1 and the saving forward); -3 elsewhere.
int launch_tokenloop_small(int m, int d, const Params& p, bool in_bf16, hipStream_t st);

// MFMA chunk path (bf16 inputs): whether (m, d, C) has a built variant, the
// workspace it needs, and the launch of the inter-chunk state-passing kernel
// followed by the read-out kernel (split schedule), or the fused kernel.
bool mfma_supported(int m, int d, int C);
// Side stream and events of the overlapped read-out (split schedule): nseg
// chunk ranges (ends in `end`), each range's read-out on `side` while the next range's state
// passing runs on the caller's stream.
constexpr int kMaxRanges = 8;
struct Overlap {
    int nseg;
    int end[kMaxRanges];  // chunk end of each range (the first starts at chunk 0)
    hipStream_t side;
    hipEvent_t ev_chain, ev_side;
};
size_t mfma_workspace_bytes(int B, int H, int T, int m, int d, int C, bool lin1, int schedule, int chain_wgs,
                            int readout_overlap);
// The split schedule's per-chunk workspace whatever the schedule choice, and
// the state-passing kernel alone (the backward takes its chunk-start states
// from it, through Params::raw).
size_t mfma_chain_workspace_bytes(int B, int H, int T, int m, int d, int C, bool lin1);
int launch_mfma_chain_only(int m, int d, const Params& p, hipStream_t st);
int launch_mfma_chunked(int m, int d, const Params& p, hipStream_t st);

// Backward of the chunk-wise forward (fp32 VALU, one workgroup per (b,h)).
// f carries the forward's inputs and shape (its state_out, y and zbuf are
// unused); the gradients are fp32 in the inputs' layouts.
struct BwdParams {
    Params f;
    const void* dy;          // [B,T,H,d], fp32 or bf16 (dy_bf16)
    const float* dstate_out; // [B,H,m,d]
    float* dq;               // [B,T,H,m]
    float* dk;               // [B,T,H,m]
    float* dv;               // [B,T,H,d]
    float* dgamma;           // [B,T,H,m] or [B,T,H]
    float* dmu;              // [B,T,H]
    float* dstate_in;        // [B,H,m,d]
    float* ws;               // bwd_workspace_bytes(...)
    int dy_bf16;
    int states_ready;        // 1: the chunk-start states are already in the workspace
    int stage_gk;            // 1: the chunk's g, kappa (and e) are staged in dynamic LDS after h
    // With states_ready: the state-passing kernel's per-chunk arrays in its
    // workspace layout ([B*H*NC][rows/16][C/16][64 lanes][4], rows = m or d):
    // g, kappa, h, e (first linearisation) and c, beta; |h|^2 as [B*H*NC][C].
    const float *chain_g, *chain_k, *chain_h, *chain_e, *chain_c, *chain_b, *chain_hh;
    // Slot rows split over split_p workgroups per sequence (1: not split).  The
    // general walk (needs the state-passing kernel's arrays): per (b,h), two
    // batch parities x split_p parts of one batch's sums over slots at xbuf, and
    // split_p progress counters at xflags.  The small-chunk walk: tagged pairs
    // at xbuf only (bwd_small_xchg_bytes).
    int split_p;
    float* xbuf;
    int* xflags;
};
size_t bwd_workspace_bytes(int B, int H, int T, int m, int d, int C);
// Workgroups per sequence of the backward (slot rows split between them), and
// the hand-off buffers that takes (0 for one).  chain: the state-passing
// kernel supplies the chunk-start states and records; chain_wgs: 0 automatic, 1 one.
int bwd_split_p(int B, int H, int m, int d, int C, bool chain, int chain_wgs);
// Whether P workgroups of m / P rows each fit the kernel's LDS budget.
bool bwd_split_fits(int m, int d, int C, int P);
size_t bwd_xchg_bytes(int B, int H, int d, int P);
int launch_bwd(int m, int d, const BwdParams& p, bool in_bf16, hipStream_t st);
// The chunk-parallel backward on the fp32 matrix cores (osr_bwd_chunk.hip):
// where it is built (m = d = C = 64, bf16 inputs, the default linearisation,
// decoding or similarity objective), with the chunk-start states already in
// the workspace (states_ready).  Same workspace layout as launch_bwd.
bool bwd_chunk_supported(int m, int d, int C, bool in_bf16, bool lin1, int mode);
int launch_bwd_chunk(int m, int d, const BwdParams& p, bool in_bf16, hipStream_t st);
// The reverse walk at small chunks (osr_bwd_small.hip): C in {1, 2, 4, 8} within
// the token loop's batch, the default linearisation, and at most 2 slot rows per
// thread on 1, 2 or 4 workgroups per sequence (bwd_small_min_p).
// Its phase 1 is the forward's small-chunk token loop with raw (and, decoding
// objective, hrec) set; f.hrec then points at those records.  Same workspace
// layout as launch_bwd, plus hrec.
// split_p = 2 or 4 splits a sequence's slot rows over that many workgroups, with their
// hand-off buffers at xbuf: per (b,h), 2 chunk parities x P parts x max(C, 8)
// tokens x (d + 4) (value, tag) pairs of 8 bytes.  At C = 16 the state-passing
// kernel is phase 1 (chunk-start states, and h in its fragment layout).
inline size_t bwd_small_xchg_bytes(int B, int H, int d, int P, int C) {
    if (P <= 1) return 0;
    return static_cast<size_t>(B) * H * 2 * P * (C > 8 ? C : 8) * (d + 4) * sizeof(uint64_t);
}
bool bwd_small_supported(int m, int d, int C, bool lin1);
int bwd_small_min_p(int m, int d, int C);
int bwd_small_split_p(int B, int H, int m, int d, int C, int chain_wgs);
int launch_bwd_small(int m, int d, const BwdParams& p, bool in_bf16, hipStream_t st);

// Layer glue (HBM-bound streaming kernels).  pre: q = conv4(xq), k = conv4(xk)
// (depthwise causal, width 4, N = H*m channels per token row), gamma =
// sigmoid(logit) (G = H*m or H values per token row), the last three raw rows
// as the next call's history.  All element buffers share the input dtype.
struct GlueParams {
    const void *xq, *xk, *glogit;    // [B,T,N], [B,T,N], [B,T,G]
    const float *wq, *wk;            // [N,4]; tap 3 weighs the current token
    const float *bq, *bk;            // [N] or null
    const void *hq_in, *hk_in;       // [B,3,N] or null (zeros)
    void *q, *k, *gamma;             // outputs, like the inputs
    void *hq_out, *hk_out;           // [B,3,N] or null
    int B, T, N, G;
    int gvec;                        // 1: G % 8 == 0 and glogit, gamma 16-byte aligned
};
// Return 0, -3 (shape outside what the kernels take) or -5 (launch error).
int launch_glue_pre(const GlueParams& p, bool in_bf16, hipStream_t st);
// out = y * GeLU(g) elementwise over n values (n % 8 == 0, 16-byte aligned).
int launch_glue_post(const void* y, bool y_bf16, const void* g, bool g_bf16, void* out, int64_t n, hipStream_t st);

}  // namespace osr
