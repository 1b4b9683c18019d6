// osr_valu.hip -- VALU (fp32) OSR kernels for gfx950: the fused single-token
// decode step and the token-by-token forward (exact recurrence at C = 1, the
// chunk-linearised recurrence at C > 1): a batched loop for chunks of 1, 2, 4
// or 8 tokens within one read-out batch, a general loop for the other sizes.
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646).  Per token, with Z the unit-projected chunk-start state
// (section "Stabilizing Memory Updates via Normalization") and S the running
// state, both m x d with row i = slot i:
//   h   = sum_i k_i z_i - v  (decoding objective), -v (similarity) or v
//         (encoding layer, subsection "Encoding layer")
//   c_i = z_i . h,  a_i = gamma_i k_i (gamma_i (c_i - k_i) for the encoding
//         layer: its per-slot error z_i . v - k_i),  w_i = max(|h|^2 - c_i^2, 0)
//   beta_i = (mu^2 + a_i^2 w_i)^(-1/2)            (eq. normalized_recurrence
//                                                  with the forget gate)
//   s_i <- beta_i (mu + a_i c_i) s_i - beta_i a_i h   (eq. recurrence_detailed;
//                                                  eq. recurrence_linear2 when
//                                                  C > 1)
//   or, with the first chunk linearisation (eq. recurrence_linear1),
//   s_i <- beta_i mu s_i + beta_i a_i c_i z_i - beta_i a_i h
//   y   = sum_i q_i s_i                           (memory read-out)
// With C = 1, Z = S and the step is the exact projected orthogonal update.
//
// Thread layout and reductions: osr_valu.h.
#include <type_traits>

#include "osr_launch.h"
#include "osr_valu.h"

namespace osr {

// One token: update the running state s from the chunk-start state z and
// return the read-out for this thread's 4 columns (valid in every thread).
// red_h and red_y must be distinct buffers, and red_y must differ from the
// red_y of the previous call (callers alternate it by token parity): that way
// one barrier per reduction orders every write after the last read of the
// same buffer.
template <class L, int D>
__device__ __forceinline__ float4 osr_token(const float4 (&z)[L::RPT], float4 (&s)[L::RPT],
                                            const TokenIn<L::RPT>& in, int mode, int lin1, float* red_h,
                                            float* red_y, int lane, int wave, int cg) {
    float4 h;
    if (mode == 0) {
        float4 hp = f4(0.f);
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) hp = fma4(in.k[i], z[i], hp);
        h = col_sum<L, D>(hp, red_h, lane, wave, cg) - in.v;
    } else if (mode == 2) {
        h = in.v;
    } else {
        h = f4(0.f) - in.v;
    }
    float cc[L::RPT + 1];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) cc[i] = dot4(z[i], h);
    cc[L::RPT] = dot4(h, h);
#pragma unroll
    for (int i = 0; i <= L::RPT; ++i) cc[i] = group_sum<L::TPR>(cc[i]);
    const float hh = cc[L::RPT];
    const float mu = in.mu;
    float4 yp = f4(0.f);
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        const float a = in.g[i] * (mode == 2 ? cc[i] - in.k[i] : in.k[i]);
        const float w = fmaxf(fmaf(-cc[i], cc[i], hh), 0.f);
        const float beta = rsqrtf(fmaf(mu, mu, a * a * w));
        const float kap = -beta * a;
        if (lin1) {
            // mu beta on the running slot, the projection term on z
            s[i] = fma4(beta * mu, s[i], fma4(beta * a * cc[i], z[i], kap * h));
        } else {
            const float gate = beta * fmaf(a, cc[i], mu);
            s[i] = fma4(gate, s[i], kap * h);
        }
        yp = fma4(in.q[i], s[i], yp);
    }
    return col_sum<L, D>(yp, red_y, lane, wave, cg);
}

// ------------------------------------------------------------------ decode --
template <int M, int D, int NT, typename TIn>
__global__ __launch_bounds__(NT) void osr_decode_kernel(Params p) {
    using L = ValuLayout<M, D, NT>;
    __shared__ float red[2][L::NW * D];
    const int bh = blockIdx.x;  // T == 1: token index b*H + h
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % L::TPR, rg = tid / L::TPR;

    const float* sin = p.state_in + static_cast<int64_t>(bh) * M * D;
    float4 s[L::RPT];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i)
        s[i] = ld_nt4(sin + (rg + L::RG * i) * D + cg * 4);
    TokenIn<L::RPT> in;
    load_token<L, M, D, TIn>(in, p, bh, rg, cg);

    project_rows<L>(s);
    float4 z[L::RPT];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) z[i] = s[i];
    const float4 y = osr_token<L, D>(z, s, in, p.mode, 0, red[0], red[1], lane, wave, cg);
    if (rg == 0) {
        float4 yg = y;
        if (p.gate) {
            const float4 g = ld4<TIn>(static_cast<const TIn*>(p.gate), static_cast<int64_t>(bh) * D + cg * 4);
            yg = make_float4(y.x * gelu(g.x), y.y * gelu(g.y), y.z * gelu(g.z), y.w * gelu(g.w));
        }
        st_y4(p.y, static_cast<int64_t>(bh) * D + cg * 4, yg, p.y_bf16);
    }

    project_rows<L>(s);
    float* sout = p.state_out + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i)
        st_nt4(sout + (rg + L::RG * i) * D + cg * 4, s[i]);
}

// -------------------------------------------------------------- token loop --
// The read-outs y do not feed back into the recurrence, so their sums over
// slots are batched: each token leaves its per-wave partials in LDS and every
// BT tokens one barrier lets the threads add them up (one float4 of the batch
// each) and store y.  With C > 1, h depends only on the chunk-start state and
// the inputs, so the chunk's h is formed up front in LDS (chunk_h) and a token
// needs no exchange across waves at all.  This loop takes the chunk sizes the
// small-chunk loop below does not (C > 1 always: C = 1 is a small chunk).
template <int M, int D, int NT, typename TIn>
__global__ __launch_bounds__(NT) void osr_tokenloop_kernel(Params p) {
    using L = ValuLayout<M, D, NT>;
    constexpr int BT = TokBatch<L>::BT, W = D + 4, Q = D / 4;
    static_assert(BT * Q <= NT, "one float4 of a batch's read-outs per thread");
    // The chunk's h and chunk_h's exchange buffers sit in dynamic LDS
    // (tokenloop_dyn_lds floats).
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    float* hbuf = dyn;                   // [C][D]
    float* redc = dyn + p.chunk * D;     // [2][BT][NW][W]
    __shared__ __attribute__((aligned(16))) float redy[2 * BT * L::NW * W];  // y batches
    const int bh = blockIdx.x;
    const int b = bh / p.H, hd = bh % p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % L::TPR, rg = tid / L::TPR;
    const int T = p.T, C = p.chunk;
    const int64_t tstride = p.H;  // consecutive tokens of one (b,h) are H rows apart

    const float* sin = p.state_in + static_cast<int64_t>(bh) * M * D;
    float4 s[L::RPT], z[L::RPT];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i)
        s[i] = *reinterpret_cast<const float4*>(sin + (rg + L::RG * i) * D + cg * 4);

    auto bth_of = [&](int t) { return (static_cast<int64_t>(b) * T + t) * p.H + hd; };
    TokenIn<L::RPT> cur, nxt;
    load_token<L, M, D, TIn>(cur, p, bth_of(0), rg, cg);
    int nredc = 0, ybatch = 0;

    for (int t = 0; t < T; ++t) {
        const int tau = t % C;
        if (tau == 0) {
            project_rows<L>(s);
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) z[i] = s[i];
            __syncthreads();  // every thread is done with the previous chunk's h
            chunk_h<L, M, D, TIn>(z, p, bth_of(t), tstride, C, p.mode, hbuf, redc, nredc, tid, lane, wave, rg, cg);
        }
        // unconditional (the last token loads itself again): a load under a branch
        // is waited for where the branch joins, which would undo the prefetch
        load_token<L, M, D, TIn>(nxt, p, bth_of(t + 1 < T ? t + 1 : t), rg, cg);

        const float4 h = *reinterpret_cast<const float4*>(hbuf + tau * D + cg * 4);
        float cc[L::RPT + 1];
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) cc[i] = dot4(z[i], h);
        cc[L::RPT] = dot4(h, h);
#pragma unroll
        for (int i = 0; i <= L::RPT; ++i) cc[i] = group_sum<L::TPR>(cc[i]);
        const float hh = cc[L::RPT];
        const float mu = cur.mu;
        float4 yp = f4(0.f);
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) {
            const float a = cur.g[i] * (p.mode == 2 ? cc[i] - cur.k[i] : cur.k[i]);
            const float w = fmaxf(fmaf(-cc[i], cc[i], hh), 0.f);
            const float beta = rsqrtf(fmaf(mu, mu, a * a * w));
            const float kap = -beta * a;
            if (p.lin1) {
                // mu beta on the running slot, the projection term on z
                s[i] = fma4(beta * mu, s[i], fma4(beta * a * cc[i], z[i], kap * h));
            } else {
                s[i] = fma4(beta * fmaf(a, cc[i], mu), s[i], kap * h);
            }
            yp = fma4(cur.q[i], s[i], yp);
        }

        // this token's read-out partial over the wave's slots, to LDS
        const int u = t % BT;
        float* rb = redy + (ybatch & 1) * (BT * L::NW * W);
        yp.x = strided_sum<L::TPR>(yp.x);
        yp.y = strided_sum<L::TPR>(yp.y);
        yp.z = strided_sum<L::TPR>(yp.z);
        yp.w = strided_sum<L::TPR>(yp.w);
        if (lane < L::TPR) *reinterpret_cast<float4*>(rb + (u * L::NW + wave) * W + cg * 4) = yp;
        if (u == BT - 1 || t == T - 1) {
            __syncthreads();  // the batch's partials visible
            const int nb = u + 1, t0 = t - u;
            if (tid < nb * Q) {
                const int uu = tid / Q, c4 = tid % Q;
                float4 acc = *reinterpret_cast<const float4*>(rb + (uu * L::NW) * W + c4 * 4);
#pragma unroll
                for (int w = 1; w < L::NW; ++w) acc = acc + *reinterpret_cast<const float4*>(rb + (uu * L::NW + w) * W + c4 * 4);
                if (p.gate) {
                    const float4 g = ld4<TIn>(static_cast<const TIn*>(p.gate), bth_of(t0 + uu) * D + c4 * 4);
                    acc = make_float4(acc.x * gelu(g.x), acc.y * gelu(g.y), acc.z * gelu(g.z), acc.w * gelu(g.w));
                }
                st_y4(p.y, bth_of(t0 + uu) * D + c4 * 4, acc, p.y_bf16);
            }
            ++ybatch;
        }
        cur = nxt;
    }
    project_rows<L>(s);
    float* sout = p.state_out + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i)
        *reinterpret_cast<float4*>(sout + (rg + L::RG * i) * D + cg * 4) = s[i];
}

// Token loop for small chunks (C = CB in {1, 2, 4, 8}, at most one batch of
// the y exchange).  Per chunk: the chunk's h over slots once (as chunk_h),
// then c, |h|^2 and the gates of all CB tokens together (CB (RPT + 1)
// independent row sums instead of RPT + 1 per token), then the CB tokens'
// state updates and read-out partials, their sums over the wave's row groups
// again together.  Every input of the next chunk (k, q, gamma, mu of its
// tokens, and the v this thread subtracts from h) is loaded while the current
// chunk computes; h alternates between two LDS buffers by chunk parity, so a
// chunk's h is written while no thread can still read the buffer (the barrier
// inside the exchange of the chunk before orders it).
// For the backward (y and state_out null, raw set): every chunk-start state
// before projection and the end state go to raw, and (decoding objective,
// hrec set) every chunk's h to hrec; the read-out is skipped.
template <int M, int D, int NT, typename TIn, int CB>
__global__ __launch_bounds__(NT) void osr_tokenloop_small_kernel(Params p) {
    using L = ValuLayout<M, D, NT>;
    constexpr int BT = TokBatch<L>::BT, W = D + 4, Q = D / 4, RPT = L::RPT;
    static_assert(CB <= BT && BT % CB == 0, "a chunk's tokens in one exchange batch");
    static_assert(BT * Q <= NT, "one float4 of a batch per thread");
    extern __shared__ __attribute__((aligned(16))) float dyn[];
    float* hbuf = dyn;                   // [2][CB][D]
    float* redc = dyn + 2 * CB * D;      // [2][BT][NW][W] the chunk's h partials
    __shared__ __attribute__((aligned(16))) float redy[2 * BT * L::NW * W];  // y batches
    const int bh = blockIdx.x;
    const int b = bh / p.H, hd = bh % p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % L::TPR, rg = tid / L::TPR;
    const int T = p.T, NCH = T / CB;
    const int mode = p.mode;
    auto bth_of = [&](int t) { return (static_cast<int64_t>(b) * T + t) * p.H + hd; };
    const TIn* kp = static_cast<const TIn*>(p.k);
    const TIn* qp = static_cast<const TIn*>(p.q);
    const TIn* gp = static_cast<const TIn*>(p.gamma);
    const TIn* mp = static_cast<const TIn*>(p.mu);
    const TIn* vp = static_cast<const TIn*>(p.v);
    // this thread's output float4 of the chunk's h: token uo, columns 4 co ..
    const int uo = tid / Q < CB ? tid / Q : CB - 1, co = tid % Q;

    const float* sin = p.state_in + static_cast<int64_t>(bh) * M * D;
    float4 s[RPT], z[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) s[i] = *reinterpret_cast<const float4*>(sin + (rg + L::RG * i) * D + cg * 4);

    // a chunk's inputs
    struct In {
        float k[CB][RPT], q[CB][RPT], g[CB][RPT], mu[CB];
        float4 vo, v[CB];
    };
    auto load_chunk = [&](In& in, int n) {
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const int64_t bt = bth_of(n * CB + u);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg + L::RG * i;
                in.k[u][i] = ld<TIn>(kp, bt * M + row);
                in.q[u][i] = ld<TIn>(qp, bt * M + row);
                in.g[u][i] = ld<TIn>(gp, p.gamma_per_slot ? bt * M + row : bt);
            }
            in.mu[u] = ld<TIn>(mp, bt);
            in.v[u] = ld4<TIn>(vp, bt * D + cg * 4);
        }
        in.vo = ld4<TIn>(vp, bth_of(n * CB + uo) * D + co * 4);
    };
    In cur, nxt;
    load_chunk(cur, 0);
    int ybatch = 0;

    float* const raw = p.raw ? p.raw + static_cast<int64_t>(bh) * p.raw_stride : nullptr;
    for (int n = 0; n < NCH; ++n) {
        if (raw) {
#pragma unroll
            for (int i = 0; i < RPT; ++i)
                *reinterpret_cast<float4*>(raw + static_cast<int64_t>(n) * M * D + (rg + L::RG * i) * D + cg * 4) = s[i];
        }
        project_rows<L>(s);
#pragma unroll
        for (int i = 0; i < RPT; ++i) z[i] = s[i];
        float* hb = hbuf + (n & 1) * (CB * D);
        // ---- the chunk's h ----
        float4 h[CB];
        if (mode == 0) {
            float* rb = redc + (n & 1) * (BT * L::NW * W);
#pragma unroll
            for (int u = 0; u < CB; ++u) {
                float4 hp = f4(0.f);
#pragma unroll
                for (int i = 0; i < RPT; ++i) hp = fma4(cur.k[u][i], z[i], hp);
                hp.x = strided_sum<L::TPR>(hp.x);
                hp.y = strided_sum<L::TPR>(hp.y);
                hp.z = strided_sum<L::TPR>(hp.z);
                hp.w = strided_sum<L::TPR>(hp.w);
                if (lane < L::TPR) *reinterpret_cast<float4*>(rb + (u * L::NW + wave) * W + cg * 4) = hp;
            }
            __syncthreads();
            if (tid < CB * Q) {
                float4 acc = *reinterpret_cast<const float4*>(rb + (uo * L::NW) * W + co * 4);
#pragma unroll
                for (int w = 1; w < L::NW; ++w) acc = acc + *reinterpret_cast<const float4*>(rb + (uo * L::NW + w) * W + co * 4);
                *reinterpret_cast<float4*>(hb + uo * D + co * 4) = acc - cur.vo;
                if (p.hrec)
                    *reinterpret_cast<float4*>(p.hrec + (static_cast<int64_t>(bh) * T + n * CB + uo) * D + co * 4) =
                        acc - cur.vo;
            }
            __syncthreads();
#pragma unroll
            for (int u = 0; u < CB; ++u) h[u] = *reinterpret_cast<const float4*>(hb + u * D + cg * 4);
        } else {
#pragma unroll
            for (int u = 0; u < CB; ++u) h[u] = mode == 2 ? cur.v[u] : f4(0.f) - cur.v[u];
        }
        // the next chunk's inputs, in flight while this one computes (the last re-reads itself)
        load_chunk(nxt, n + 1 < NCH ? n + 1 : n);

        // ---- c, |h|^2 and the gates of every token of the chunk ----
        float cc[CB][RPT + 1];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) cc[u][i] = dot4(z[i], h[u]);
            cc[u][RPT] = dot4(h[u], h[u]);
        }
#pragma unroll
        for (int u = 0; u < CB; ++u)
#pragma unroll
            for (int i = 0; i <= RPT; ++i) cc[u][i] = group_sum<L::TPR>(cc[u][i]);
        // ---- the tokens in turn: state update, read-out partial ----
        float4 yp[CB];
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            const float hh = cc[u][RPT], mu = cur.mu[u];
            yp[u] = f4(0.f);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float a = cur.g[u][i] * (mode == 2 ? cc[u][i] - cur.k[u][i] : cur.k[u][i]);
                const float w = fmaxf(fmaf(-cc[u][i], cc[u][i], hh), 0.f);
                const float beta = rsqrtf(fmaf(mu, mu, a * a * w));
                const float kap = -beta * a;
                if (p.lin1) {
                    s[i] = fma4(beta * mu, s[i], fma4(beta * a * cc[u][i], z[i], kap * h[u]));
                } else {
                    s[i] = fma4(beta * fmaf(a, cc[u][i], mu), s[i], kap * h[u]);
                }
                yp[u] = fma4(cur.q[u][i], s[i], yp[u]);
            }
        }
        if (!p.y) {
            cur = nxt;
            continue;
        }
        float* rb = redy + (ybatch & 1) * (BT * L::NW * W);
        const int u0 = (n * CB) % BT;  // this chunk's first slot in the y batch
#pragma unroll
        for (int u = 0; u < CB; ++u) {
            yp[u].x = strided_sum<L::TPR>(yp[u].x);
            yp[u].y = strided_sum<L::TPR>(yp[u].y);
            yp[u].z = strided_sum<L::TPR>(yp[u].z);
            yp[u].w = strided_sum<L::TPR>(yp[u].w);
        }
        if (lane < L::TPR)
#pragma unroll
            for (int u = 0; u < CB; ++u) *reinterpret_cast<float4*>(rb + ((u0 + u) * L::NW + wave) * W + cg * 4) = yp[u];
        const int tend = (n + 1) * CB;  // tokens done
        if (tend % BT == 0 || n + 1 == NCH) {
            __syncthreads();  // the batch's partials visible
            const int nb = u0 + CB, t0 = tend - nb;
            if (tid < nb * Q) {
                const int uu = tid / Q, c4 = tid % Q;
                float4 acc = *reinterpret_cast<const float4*>(rb + (uu * L::NW) * W + c4 * 4);
#pragma unroll
                for (int w = 1; w < L::NW; ++w) acc = acc + *reinterpret_cast<const float4*>(rb + (uu * L::NW + w) * W + c4 * 4);
                if (p.gate) {
                    const float4 g = ld4<TIn>(static_cast<const TIn*>(p.gate), bth_of(t0 + uu) * D + c4 * 4);
                    acc = make_float4(acc.x * gelu(g.x), acc.y * gelu(g.y), acc.z * gelu(g.z), acc.w * gelu(g.w));
                }
                st_y4(p.y, bth_of(t0 + uu) * D + c4 * 4, acc, p.y_bf16);
            }
            ++ybatch;
        }
        cur = nxt;
    }
    if (raw) {
#pragma unroll
        for (int i = 0; i < RPT; ++i)
            *reinterpret_cast<float4*>(raw + static_cast<int64_t>(NCH) * M * D + (rg + L::RG * i) * D + cg * 4) = s[i];
    }
    if (!p.state_out) return;
    project_rows<L>(s);
    float* sout = p.state_out + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < RPT; ++i) *reinterpret_cast<float4*>(sout + (rg + L::RG * i) * D + cg * 4) = s[i];
}

// Dynamic LDS of the general token loop (floats).
template <int M, int D, int NT>
static size_t tokenloop_dyn_lds(int C) {
    using L = ValuLayout<M, D, NT>;
    return static_cast<size_t>(C) * D + 2 * TokBatch<L>::BT * L::NW * (D + 4);
}

// ----------------------------------------------------------------- launch --
template <int M, int D>
// small_only: the small-chunk loop at C in {1, 2, 4, 8} (the backward's phase 1,
// which stores the chunk-start states), or -3 where it does not apply.
static int launch_valu_md(bool decode, const Params& p, bool in_bf16, hipStream_t st, bool small_only = false) {
    constexpr int TPR = D / 4;
    // Decode: up to 8 waves per state (fewer rows per thread: ~100 VGPRs, 4 waves per SIMD), which
    // shortens each workgroup's arithmetic between its state load and store; measured 9% faster
    // than 4 waves at m = d = 128.
    constexpr int NT_DEC = (M * TPR < 512) ? M * TPR : 512;
    constexpr int NT_TOK = tokenloop_threads<M, D>();
    const dim3 grid(static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H));
    if (decode) {
        if (in_bf16)
            hipLaunchKernelGGL((osr_decode_kernel<M, D, NT_DEC, uint16_t>), grid, dim3(NT_DEC), 0, st, p);
        else
            hipLaunchKernelGGL((osr_decode_kernel<M, D, NT_DEC, float>), grid, dim3(NT_DEC), 0, st, p);
    } else {
        // small chunks that fit one exchange batch: the batched loop
        constexpr int BT = TokBatch<ValuLayout<M, D, NT_TOK>>::BT;
        const int C = p.chunk;
        if ((C == 1 || C == 2 || C == 4 || C == 8) && C <= BT) {
            using L = ValuLayout<M, D, NT_TOK>;
            const size_t lds = (2 * static_cast<size_t>(C) * D + 2 * BT * L::NW * (D + 4)) * sizeof(float);
            auto go = [&](auto cb) {
                constexpr int CBV = decltype(cb)::value;
                if constexpr (CBV <= BT) {
                    if (in_bf16)
                        hipLaunchKernelGGL((osr_tokenloop_small_kernel<M, D, NT_TOK, uint16_t, CBV>), grid, dim3(NT_TOK),
                                           lds, st, p);
                    else
                        hipLaunchKernelGGL((osr_tokenloop_small_kernel<M, D, NT_TOK, float, CBV>), grid, dim3(NT_TOK), lds,
                                           st, p);
                }
            };
            if (C == 1)
                go(std::integral_constant<int, 1>{});
            else if (C == 2)
                go(std::integral_constant<int, 2>{});
            else if (C == 4)
                go(std::integral_constant<int, 4>{});
            else
                go(std::integral_constant<int, 8>{});
            return hipGetLastError() == hipSuccess ? 0 : -5;
        }
        if (small_only || C < 2) return -3;
        const size_t lds = tokenloop_dyn_lds<M, D, NT_TOK>(p.chunk) * sizeof(float);
        if (in_bf16)
            hipLaunchKernelGGL((osr_tokenloop_kernel<M, D, NT_TOK, uint16_t>), grid, dim3(NT_TOK), lds, st, p);
        else
            hipLaunchKernelGGL((osr_tokenloop_kernel<M, D, NT_TOK, float>), grid, dim3(NT_TOK), lds, st, p);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int M>
static int launch_valu_m(bool decode, int d, const Params& p, bool in_bf16, hipStream_t st, bool small_only = false) {
    switch (d) {
        case 16: return launch_valu_md<M, 16>(decode, p, in_bf16, st, small_only);
        case 32: return launch_valu_md<M, 32>(decode, p, in_bf16, st, small_only);
        case 64: return launch_valu_md<M, 64>(decode, p, in_bf16, st, small_only);
        case 128: return launch_valu_md<M, 128>(decode, p, in_bf16, st, small_only);
        default: return -3;
    }
}

int launch_valu(bool decode, int m, int d, const Params& p, bool in_bf16, hipStream_t st) {
    switch (m) {
        case 16: return launch_valu_m<16>(decode, d, p, in_bf16, st);
        case 32: return launch_valu_m<32>(decode, d, p, in_bf16, st);
        case 64: return launch_valu_m<64>(decode, d, p, in_bf16, st);
        case 128: return launch_valu_m<128>(decode, d, p, in_bf16, st);
        default: return -3;
    }
}

int launch_tokenloop_small(int m, int d, const Params& p, bool in_bf16, hipStream_t st) {
    switch (m) {
        case 16: return launch_valu_m<16>(false, d, p, in_bf16, st, true);
        case 32: return launch_valu_m<32>(false, d, p, in_bf16, st, true);
        case 64: return launch_valu_m<64>(false, d, p, in_bf16, st, true);
        case 128: return launch_valu_m<128>(false, d, p, in_bf16, st, true);
        default: return -3;
    }
}

}  // namespace osr
