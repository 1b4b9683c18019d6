// osr_bwd_kernel.h -- backward of the chunk-wise OSR forward on gfx950 (fp32 VALU).
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646).  The layer is trained through its chunk-wise form (section
// "Parallel and Hardware Efficient Form", eq. recurrence_linear2); this kernel
// returns the vector-Jacobian product of that forward at chunk size C (exact
// recurrence at C = 1): given dy and the gradient of the returned state, the
// gradients of q, k, v, gamma, mu and the initial state.  The first chunk
// linearisation (eq. recurrence_linear1: gate mu beta, and the projection term
// beta a c on the chunk-start slot z) is handled by the same walk, with one
// more adjoint per slot, de_i = z_i . D_i, and the term's share of dZ.
//
// Forward per token t of a chunk (Z = unit-projected chunk-start state, R the
// running state, rows = slots):
//   h = sum_i k_i z_i - v | -v | v      c_i = z_i . h      hh = |h|^2
//   a_i = gamma_i k_i (encoding layer: gamma_i (c_i - k_i))
//   w_i = max(hh - c_i^2, 0)            beta_i = (mu^2 + a_i^2 w_i)^(-1/2)
//   g_i = beta_i (mu + a_i c_i)         kap_i = -beta_i a_i
//   r_i <- g_i r_i + kap_i h            y = sum_i q_i r_i
// Reverse of one token, with D the gradient of the state after the token:
//   dq_i = r_i . dy;  D_i += q_i dy
//   dg_i = r_prev_i . D_i;  dkap_i = h . D_i
//   (beta, a, c, mu) from (dg, dkap) by the chain rule through g and kap,
//   then through beta = (mu^2 + a^2 w)^(-1/2) and w (only where w > 0)
//   dh = sum_i (kap_i D_i + dc_i z_i) + 2 h dhh
//   dZ_i += dc_i h (+ k_i dh, decoding objective: dk_i += z_i . dh)
//   dv = -dh (decoding, similarity) or dh (encoding layer)
//   D_i <- g_i D_i  (the gradient of the state before the token)
// At the chunk start dZ + D (the gradient of Z) goes back through the
// projection onto the sphere: dS_i = (dz_i - z_i (z_i . dz_i)) / |s_i|.
//
// Inside a chunk neither h (it depends on Z and the inputs only) nor any of the
// reverse walk's sums over slots feeds back into the state recurrence, which
// is elementwise per slot.  So the sums over slots, the only reductions that
// cross waves, are batched: h for a batch of BT tokens in one LDS exchange, and
// in the reverse walk the per-token partials of dh (with d|h|^2, dmu and a
// per-token dgamma) for BT tokens in another.  In both, the sums over waves
// are spread over the threads (one float4 of the batch each) rather than
// repeated by every thread.  The per-token steps in between
// reduce only over d, inside a row group (DPP).
//
// One workgroup per (b,h), state in registers in the layout of osr_valu.h.
// Phase 1 runs the forward and keeps every chunk-start state (before
// projection) in the workspace, unless the matrix-core state-passing kernel
// has already stored them there (states_ready).  Phase 2 walks the chunks
// backwards: it forms the chunk's h in LDS, runs the chunk forward again from
// its stored start (keeping the state before each token and the per-token c,
// beta, |h|^2 in the workspace), then walks the chunk's tokens backwards.
#pragma once

#include "osr_launch.h"
#include "osr_valu.h"

namespace osr {

typedef unsigned int bwd_u32x4 __attribute__((ext_vector_type(4)));

// Per-token record kept for the reverse walk: c[M], beta[M], |h|^2, pad.
template <int M, int D>
struct TokRec {
    static constexpr int C_OFF = 0, B_OFF = M, HH_OFF = 2 * M;
    static constexpr int SIZE = 2 * M + 4;
};

template <int M, int D>
__host__ __device__ inline int64_t bwd_floats_per_bh(int T, int C) {
    return (static_cast<int64_t>(T / C) + 1 + C) * M * D + static_cast<int64_t>(C) * TokRec<M, D>::SIZE;
}

// One forward token given its h: updates r, returns the per-slot c and beta
// and |h|^2 (valid in every thread of a row group).  No cross-wave exchange.
// LIN1: the first chunk linearisation, r_i <- mu beta_i r_i + beta_i a_i c_i z_i
// + kap_i h (eq. recurrence_linear1).
template <class L, bool LIN1>
__device__ __forceinline__ void fwd_token_h(const float4 (&z)[L::RPT], float4 (&r)[L::RPT], const float (&k)[L::RPT],
                                            const float (&g)[L::RPT], float mu, float4 h, int mode,
                                            float (&c)[L::RPT], float (&beta)[L::RPT], float& hh) {
    float cc[L::RPT + 1];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) cc[i] = dot4(z[i], h);
    cc[L::RPT] = dot4(h, h);
#pragma unroll
    for (int i = 0; i <= L::RPT; ++i) cc[i] = group_sum<L::TPR>(cc[i]);
    hh = cc[L::RPT];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        const float a = g[i] * (mode == 2 ? cc[i] - k[i] : k[i]);
        const float w = fmaxf(fmaf(-cc[i], cc[i], hh), 0.f);
        const float b = rsqrtf(fmaf(mu, mu, a * a * w));
        if constexpr (LIN1)
            r[i] = fma4(b * mu, r[i], fma4(b * a * cc[i], z[i], (-b * a) * h));
        else
            r[i] = fma4(b * fmaf(a, cc[i], mu), r[i], (-b * a) * h);
        c[i] = cc[i];
        beta[i] = b;
    }
}

// k, gamma (per slot row of this thread) and mu of one token.
template <class L, int M, typename TIn>
__device__ __forceinline__ void load_kgm(const Params& f, int64_t bth, int rg, float (&k)[L::RPT],
                                         float (&g)[L::RPT], float& mu) {
    const TIn* kp = static_cast<const TIn*>(f.k);
    const TIn* gp = static_cast<const TIn*>(f.gamma);
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        const int row = rg + L::RG * i;
        k[i] = ld<TIn>(kp, bth * M + row);
        g[i] = ld<TIn>(gp, f.gamma_per_slot ? bth * M + row : bth);  // one load, no branch
    }
    mu = ld<TIn>(static_cast<const TIn*>(f.mu), bth);
}

// What the reverse walk reads for one token besides h: its inputs, its
// record, dy and (PF_STATE) the state before it.
template <int RPT>
struct RevIn {
    TokenIn<RPT> in;
    float c[RPT], beta[RPT];
    float hh;
    float4 dy;
    float4 rp[RPT];
};

// Offset of (row, token tau) in one chunk's per-slot array of the state-passing
// kernel's workspace: lane (lg, lc) of the fragment for row block row/16 and
// token tile tau/16 holds row 16 (row/16) + lc at tokens 16 (tau/16) + 4 lg .. +3.
__device__ __forceinline__ int64_t gate_frag(int row, int tau, int C) {
    return ((static_cast<int64_t>(row >> 4) * (C >> 4) + (tau >> 4)) * 64 + ((tau & 15) >> 2) * 16 + (row & 15)) * 4 +
           (tau & 3);
}

// ch: this (b,h)'s chunk index b*H*NC + n, for the state-passing kernel's
// records (chain_c set); otherwise the records are the kernel's own (trec).
template <class L, int M, int D, typename TIn, bool PF_STATE, bool DYB>
__device__ __forceinline__ void load_rev(RevIn<L::RPT>& x, const BwdParams& p, const float* trec,
                                         const float* rtok, int64_t bth, int64_t ch, int tau, int rg, int cg,
                                         int el0) {
    using TR = TokRec<M, D>;
    load_token<L, M, D, TIn>(x.in, p.f, bth, rg, cg);
    // c, beta and |h|^2 from the state-passing kernel's arrays or from this
    // kernel's own records: the source is chosen by address, not by branch,
    // so each value is one load whose wait can trail it (a load on either arm
    // of a branch is waited for where the arms join)
    const int C = p.f.chunk;
    const bool chain = p.chain_c != nullptr;
    const float* rec = trec + static_cast<int64_t>(tau) * TR::SIZE;
    const float* cc = chain ? p.chain_c + ch * M * C : rec + TR::C_OFF;
    const float* cb = chain ? p.chain_b + ch * M * C : rec + TR::B_OFF;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        const int row = rg + L::RG * i;
        const int64_t o = chain ? gate_frag(row, tau, C) : row;
        x.c[i] = cc[o];
        x.beta[i] = cb[o];
    }
    x.hh = *(chain ? p.chain_hh + ch * C + tau : rec + TR::HH_OFF);
    if constexpr (DYB)
        x.dy = ld4<uint16_t>(static_cast<const uint16_t*>(p.dy), bth * D + cg * 4);
    else
        x.dy = ld4<float>(static_cast<const float*>(p.dy), bth * D + cg * 4);
    if constexpr (PF_STATE) {
        const float* rpre = rtok + static_cast<int64_t>(tau) * M * D;
#pragma unroll
        for (int i = 0; i < L::RPT; ++i)
            x.rp[i] = *reinterpret_cast<const float4*>(rpre + el0 + i * L::RG * D);
    }
}

// P > 1: the slot rows of a sequence split over P workgroups (M / P rows
// each); they exchange each batch's sums over slots (below).  Only with the
// state-passing kernel's chunk-start states and records (the host ensures it).
// Split workgroups (P > 1, at most 32 rows, 2 per thread): the chunk's per-row
// records of this workgroup's rows, and (d <= 64) the chunk's dy, are staged
// in LDS at the chunk start, all loads in flight at once, so that per token
// only the state before the token comes from memory (from L2, where the
// chunk's rerun left it).  Layout, floats: [5][C][ML] c, beta, k, q, gamma (per
// slot); [3][C] mu, |h|^2, gamma (per token); then (d <= 64) [C][D] dy.
template <int ML, int D>
struct StagedRec {
    static constexpr int A_C = 0, A_B = 1, A_K = 2, A_Q = 3, A_G = 4;
    static constexpr bool DY = D <= 64;
    __host__ __device__ static constexpr int64_t floats(int C) {
        return (5 * static_cast<int64_t>(ML) + 3) * C + (DY ? static_cast<int64_t>(C) * D : 0);
    }
};

template <class L, int ML, int D, bool DYB>
__device__ __forceinline__ void load_rev_staged(RevIn<L::RPT>& x, const BwdParams& p, const float* srec,
                                                const float* rpre, int64_t bth, int tau, int rgl, int cg, int el0) {
    using SR = StagedRec<ML, D>;
    const int C = p.f.chunk;
    const float* tok = srec + 5 * static_cast<int64_t>(ML) * C;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        const int rl = rgl + L::RG * i;
        x.c[i] = srec[(SR::A_C * C + tau) * ML + rl];
        x.beta[i] = srec[(SR::A_B * C + tau) * ML + rl];
        x.in.k[i] = srec[(SR::A_K * C + tau) * ML + rl];
        x.in.q[i] = srec[(SR::A_Q * C + tau) * ML + rl];
        // (a per-token gamma: its own array, selected by address)
        x.in.g[i] = (p.f.gamma_per_slot ? srec + (SR::A_G * C + tau) * ML + rl : tok + 2 * C + tau)[0];
    }
    x.in.mu = tok[tau];
    x.hh = tok[C + tau];
    if constexpr (SR::DY)
        x.dy = *reinterpret_cast<const float4*>(tok + 3 * C + tau * D + cg * 4);
    else if constexpr (DYB)
        x.dy = ld4<uint16_t>(static_cast<const uint16_t*>(p.dy), bth * D + cg * 4);
    else
        x.dy = ld4<float>(static_cast<const float*>(p.dy), bth * D + cg * 4);
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) x.rp[i] = *reinterpret_cast<const float4*>(rpre + el0 + i * L::RG * D);
}

// Batches of the reverse walk's exchange over slots.  The token loop's batch
// (TokBatch, also the chunk's h here) is capped at 4 tokens at d = 128 for its
// LDS; where the split walk stages its records (P > 1, at most 32 rows and 2
// per thread) at d = 128 it takes 8 tokens, which halves the hand-offs between
// its workgroups, in one exchange buffer instead of two alternating ones (the
// barrier that publishes a batch's sums already orders every read of the
// buffer before the next batch's writes).
template <int M, int D, int NT, int P>
struct WalkBatch {
    using L = ValuLayout<M / P, D, NT>;
    static constexpr bool STG = P > 1 && L::RPT <= 2 && M / P <= 32;
    static constexpr int BTC = TokBatch<L>::BT;                      // chunk_h's batch
    static constexpr int BT = (STG && L::TPR == 32 && BTC < 8) ? 8 : BTC;
    static constexpr bool RED2 = 2 * BTC >= 2 * BT;                // two alternating buffers
    static constexpr int RED = (2 * BTC > BT ? 2 * BTC : BT) * L::NW * (D + 4);  // red floats
    static constexpr int TOT = BT * (D + 4);                         // tot floats
};

template <int M, int D, int NT, typename TIn, bool LIN1, bool DYB, int P = 1>
__global__ __launch_bounds__(NT) void osr_bwd_kernel(BwdParams p) {
    static_assert(P == 1 || (M / P >= 16 && sizeof(TIn) == 2), "split: bf16 inputs, 16 rows or more each");
    using L = ValuLayout<M / P, D, NT>;
    using TR = TokRec<M, D>;
    using WB = WalkBatch<M, D, NT, P>;
    constexpr int BT = WB::BT, W = D + 4;
    // The reverse walk loads the next token's inputs and record while it works on
    // the current one, and the state before it too, where registers allow.
    constexpr bool PF_TOKEN = L::RPT <= 4;
    constexpr bool PF_STATE = L::RPT <= 2;
    // Two token buffers used in turn (no register copy of loads in flight) where
    // registers allow; at 4 slot rows per thread the second buffer spilled.
    constexpr bool DBUF = L::RPT <= 2;
    extern __shared__ __attribute__((aligned(16))) float hbuf[];  // [C][D], dynamic
    float* const gst = hbuf + p.f.chunk * D;  // [2 or 3][M*C]: staged gates (stage_gk)
    float* const srec = gst + (p.stage_gk ? (LIN1 ? 3 : 2) * M * p.f.chunk : 0);  // StagedRec (STG)
    __shared__ __attribute__((aligned(16))) float red[WB::RED];
    __shared__ __attribute__((aligned(16))) float tot[WB::TOT];  // a batch's sums over slots
    static_assert(BT * (D / 4 + 1) <= NT, "one float4 of a batch's sums per thread");
    const int bh = P > 1 ? blockIdx.x / P : blockIdx.x;
    const int pidx = P > 1 ? blockIdx.x % P : 0;  // this workgroup's rows: [pidx M/P, (pidx + 1) M/P)
    const int b = bh / p.f.H, hd = bh % p.f.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // rg: the (global) slot row of this thread's first row
    const int cg = tid % L::TPR, rgl = tid / L::TPR, rg = pidx * (M / P) + rgl;
    constexpr int ML = M / P;
    // staged records (StagedRec): at most 32 rows and 2 rows per thread (more spilled)
    constexpr bool STG = WB::STG;
    static_assert(STG == (P > 1 && L::RPT <= 2 && ML <= 32), "staging rule");
    const int T = p.f.T, C = p.f.chunk, NC = T / C;
    const int mode = p.f.mode;
    const bool enc = !STG && mode == 2;  // (the split path never runs the encoding layer)
    const int64_t tstride = p.f.H;  // consecutive tokens of one (b,h) are H rows apart

    float* ws = p.ws + static_cast<int64_t>(bh) * bwd_floats_per_bh<M, D>(T, C);
    float* sck = ws;                                          // [NC+1][M][D]
    float* rtok = sck + static_cast<int64_t>(NC + 1) * M * D;  // [C][M][D]
    float* trec = rtok + static_cast<int64_t>(C) * M * D;      // [C][TR::SIZE]
    auto el = [&](int i) { return (rg + L::RG * i) * D + cg * 4; };  // this thread's state elements
    auto bth_of = [&](int t) { return (static_cast<int64_t>(b) * T + t) * p.f.H + hd; };
    int nred = 0;  // LDS exchanges so far: consecutive ones use alternate halves of red
    int nbatch = 0;  // batches exchanged with the other workgroups (P > 1)
    bool xbroken = false;  // a wait for them gave up (then the results are wrong, but every wave ends)

    // ---- phase 1: forward, keeping every chunk-start state ----
    // (skipped when the state-passing kernel has stored them: then only the end
    // state is read back)
    float4 r[L::RPT], z[L::RPT];
    const float* sin = p.states_ready ? sck + static_cast<int64_t>(NC) * M * D
                                      : p.f.state_in + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) r[i] = *reinterpret_cast<const float4*>(sin + el(i));
    for (int n = 0; n < (p.states_ready ? 0 : NC); ++n) {
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) *reinterpret_cast<float4*>(sck + static_cast<int64_t>(n) * M * D + el(i)) = r[i];
        project_rows<L>(r);
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) z[i] = r[i];
        __syncthreads();  // every thread is done with the previous chunk's hbuf
        chunk_h<L, M, D, TIn>(z, p.f, bth_of(n * C), tstride, C, mode, hbuf, red, nred, tid, lane, wave, rg, cg);
        float kc[L::RPT], gc[L::RPT], muc, kn[L::RPT], gn[L::RPT], mun;
        load_kgm<L, M, TIn>(p.f, bth_of(n * C), rg, kc, gc, muc);
        for (int tau = 0; tau < C; ++tau) {
            // unconditional (the last token loads itself again): no load under a branch
            load_kgm<L, M, TIn>(p.f, bth_of(n * C + (tau + 1 < C ? tau + 1 : tau)), rg, kn, gn, mun);
            const float4 h = *reinterpret_cast<const float4*>(hbuf + tau * D + cg * 4);
            float c[L::RPT], beta[L::RPT], hh;
            fwd_token_h<L, LIN1>(z, r, kc, gc, muc, h, mode, c, beta, hh);
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) {
                kc[i] = kn[i];
                gc[i] = gn[i];
            }
            muc = mun;
        }
    }
    if (!p.states_ready) {
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) *reinterpret_cast<float4*>(sck + static_cast<int64_t>(NC) * M * D + el(i)) = r[i];
    }

    // ---- the returned state is the end state projected: its backward ----
    float4 dR[L::RPT];
    {
        const float* dso = p.dstate_out + static_cast<int64_t>(bh) * M * D;
        float n2[L::RPT], pr[L::RPT];
        float4 o[L::RPT];
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) {
            dR[i] = *reinterpret_cast<const float4*>(dso + el(i));
            n2[i] = group_sum<L::TPR>(dot4(r[i], r[i]));
            o[i] = rsqrtf(n2[i]) * r[i];
            pr[i] = group_sum<L::TPR>(dot4(o[i], dR[i]));
        }
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) dR[i] = rsqrtf(n2[i]) * fma4(-pr[i], o[i], dR[i]);
    }

    // ---- phase 2: chunks in reverse ----
    for (int n = NC - 1; n >= 0; --n) {
        float inv[L::RPT];
        {
            const float* s0 = sck + static_cast<int64_t>(n) * M * D;
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) {
                r[i] = *reinterpret_cast<const float4*>(s0 + el(i));
                inv[i] = rsqrtf(group_sum<L::TPR>(dot4(r[i], r[i])));
                r[i] = inv[i] * r[i];
                z[i] = r[i];
            }
        }
        __syncthreads();  // the previous chunk's reverse walk is done with hbuf, red and the records
        if (p.stage_gk) {
            // the chunk's g, kappa (and e) into LDS, all loads of a round in flight
            // before any LDS write; visible after the barrier that ends the h step below
            const int64_t chs = (static_cast<int64_t>(bh) * NC + n) * M * C;
            const int n4 = M * C / 4, narr = LIN1 ? 3 : 2;
            const float* src[3] = {p.chain_g + chs, p.chain_k + chs, LIN1 ? p.chain_e + chs : p.chain_g + chs};
            for (int base = tid; base < n4; base += 2 * NT) {
                float4 v[3][2];
#pragma unroll
                for (int a = 0; a < 3; ++a)
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const int idx = min(base + j * NT, n4 - 1);
                        if (a < narr) v[a][j] = reinterpret_cast<const float4*>(src[a])[idx];
                    }
#pragma unroll
                for (int a = 0; a < 3; ++a)
#pragma unroll
                    for (int j = 0; j < 2; ++j)
                        if (a < narr && base + j * NT < n4)
                            reinterpret_cast<float4*>(gst + a * M * C)[base + j * NT] = v[a][j];
            }
        }
        if constexpr (STG) {
            // this workgroup's rows of the chunk's records (and dy): 8 loads in flight per
            // thread before any LDS write (clamped, unconditional); visible after the
            // barrier that ends the h step below
            using SR = StagedRec<ML, D>;
            const int64_t chc = (static_cast<int64_t>(bh) * NC + n) * M * C;
            const int row0 = pidx * ML;
            constexpr int G8 = 8;
            // fp32 sources: c, beta [2][C][ML] (the state-passing kernel's arrays), |h|^2 [C]
            const int nf = 2 * ML * C + C;
            for (int base = tid; base < nf; base += G8 * NT) {
                float v[G8];
#pragma unroll
                for (int g = 0; g < G8; ++g) {
                    const int idx = min(base + g * NT, nf - 1);
                    const int a = idx / (ML * C), r = idx % (ML * C);
                    const float* src = a == 0   ? p.chain_c + chc + gate_frag(row0 + r % ML, r / ML, C)
                                       : a == 1 ? p.chain_b + chc + gate_frag(row0 + r % ML, r / ML, C)
                                                : p.chain_hh + (static_cast<int64_t>(bh) * NC + n) * C + (idx - 2 * ML * C);
                    v[g] = *src;
                }
#pragma unroll
                for (int g = 0; g < G8; ++g) {
                    const int idx = base + g * NT;
                    if (idx < nf) srec[idx < 2 * ML * C ? idx : 5 * ML * C + C + (idx - 2 * ML * C)] = v[g];
                }
            }
            // input sources: k, q, gamma [3][C][ML], then mu and a per-token gamma [2][C]
            const int ni = 3 * ML * C + 2 * C;
            const TIn* kp = static_cast<const TIn*>(p.f.k);
            const TIn* qp = static_cast<const TIn*>(p.f.q);
            const TIn* gp = static_cast<const TIn*>(p.f.gamma);
            const TIn* mp = static_cast<const TIn*>(p.f.mu);
            for (int base = tid; base < ni; base += G8 * NT) {
                float v[G8];
#pragma unroll
                for (int g = 0; g < G8; ++g) {
                    const int idx = min(base + g * NT, ni - 1);
                    const TIn* src;
                    if (idx < 3 * ML * C) {
                        const int a = idx / (ML * C), r = idx % (ML * C);
                        const int64_t bt = bth_of(n * C + r / ML), o = bt * M + row0 + r % ML;
                        // (a per-token gamma has no per-slot array: the token's value stands in)
                        src = a == 0 ? kp + o : a == 1 ? qp + o : gp + (p.f.gamma_per_slot ? o : bt);
                    } else {
                        const int j = idx - 3 * ML * C;
                        const int64_t bt = bth_of(n * C + j % C);
                        src = j < C ? mp + bt : gp + (p.f.gamma_per_slot ? bt * M : bt);
                    }
                    v[g] = ld<TIn>(src, 0);
                }
#pragma unroll
                for (int g = 0; g < G8; ++g) {
                    const int idx = base + g * NT;
                    if (idx < ni) {
                        const int j = idx - 3 * ML * C;  // (the tail: mu, then a per-token gamma)
                        srec[idx < 3 * ML * C ? 2 * ML * C + idx : 5 * ML * C + (j < C ? j : 2 * C + (j - C))] = v[g];
                    }
                }
            }
            if constexpr (SR::DY) {
                // the chunk's dy [C][D] (fp32 in LDS), float4 pieces
                float* sdy = srec + 5 * ML * C + 3 * C;
                const int n4 = C * D / 4;
                for (int base = tid; base < n4; base += G8 * NT) {
                    float4 v[G8];
#pragma unroll
                    for (int g = 0; g < G8; ++g) {
                        const int idx = min(base + g * NT, n4 - 1);
                        const int64_t o = bth_of(n * C + idx / (D / 4)) * D + (idx % (D / 4)) * 4;
                        if constexpr (DYB)
                            v[g] = ld4<uint16_t>(static_cast<const uint16_t*>(p.dy), o);
                        else
                            v[g] = ld4<float>(static_cast<const float*>(p.dy), o);
                    }
#pragma unroll
                    for (int g = 0; g < G8; ++g)
                        if (base + g * NT < n4) reinterpret_cast<float4*>(sdy)[base + g * NT] = v[g];
                }
            }
        }
        if (p.chain_h && mode == 0) {
            // the chunk's h as the state-passing kernel formed it (lane (lg, lc) of the
            // fragment for column block jb and token tile tb holds h[16tb + 4lg + r][16jb + lc])
            const float* hs = p.chain_h + (static_cast<int64_t>(bh) * NC + n) * D * C;
            // 8 loads in flight per thread before any LDS write (clamped, unconditional)
            constexpr int G8 = 8;
            for (int base = tid; base < C * D; base += G8 * NT) {
                float hv[G8];
#pragma unroll
                for (int g = 0; g < G8; ++g) {
                    const int idx = min(base + g * NT, C * D - 1);
                    const int tau = idx / D, j = idx % D;
                    const int lane_f = ((tau & 15) >> 2) * 16 + (j & 15);
                    hv[g] = hs[((static_cast<int64_t>(j >> 4) * (C >> 4) + (tau >> 4)) * 64 + lane_f) * 4 + (tau & 3)];
                }
#pragma unroll
                for (int g = 0; g < G8; ++g)
                    if (base + g * NT < C * D) hbuf[base + g * NT] = hv[g];
            }
            __syncthreads();
        } else {
            chunk_h<L, M, D, TIn>(z, p.f, bth_of(n * C), tstride, C, mode, hbuf, red, nred, tid, lane, wave, rg,
                                  cg);
        }

        const int64_t ch = static_cast<int64_t>(bh) * NC + n;
        // forward again over the chunk, keeping what the reverse walk needs
        if (p.chain_c) {
            // elementwise, from the state-passing kernel's gates of this chunk, staged in
            // LDS above when they fit (read from memory, each token's gates cost one load
            // latency, as the rerun's work per token is small).  One copy of the loop per
            // source, so each reads through a pointer of one address space.
            auto rerun = [&](const float* gch, const float* kch, const float* ech) __attribute__((always_inline)) {
                float gcur[L::RPT], kcur[L::RPT], ecur[L::RPT] = {}, gnx[L::RPT], knx[L::RPT], enx[L::RPT] = {};
                auto load_g = [&](int tau, float (&g)[L::RPT], float (&k)[L::RPT], float (&e)[L::RPT]) {
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i) {
                        const int64_t o = gate_frag(rg + L::RG * i, tau, C);
                        g[i] = gch[o];
                        k[i] = kch[o];
                        if constexpr (LIN1) e[i] = ech[o];
                    }
                };
                load_g(0, gcur, kcur, ecur);
                for (int tau = 0; tau < C; ++tau) {
                    // the next token's loads go first, unconditionally (the last token loads
                    // itself again): a wave's memory counter drains in issue order, so the
                    // wait for them then covers no store of this token, and none of them
                    // sits under a branch (waited for where the branch joins)
                    load_g(tau + 1 < C ? tau + 1 : tau, gnx, knx, enx);
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i)
                        *reinterpret_cast<float4*>(rtok + static_cast<int64_t>(tau) * M * D + el(i)) = r[i];
                    const float4 h = *reinterpret_cast<const float4*>(hbuf + tau * D + cg * 4);
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i) {
                        if constexpr (LIN1)
                            r[i] = fma4(gcur[i], r[i], fma4(ecur[i], z[i], kcur[i] * h));
                        else
                            r[i] = fma4(gcur[i], r[i], kcur[i] * h);
                        gcur[i] = gnx[i];
                        kcur[i] = knx[i];
                        if constexpr (LIN1) ecur[i] = enx[i];
                    }
                }
            };
            if (p.stage_gk)
                rerun(gst, gst + M * C, gst + 2 * M * C);
            else
                rerun(p.chain_g + ch * M * C, p.chain_k + ch * M * C, LIN1 ? p.chain_e + ch * M * C : p.chain_g);
        } else {
            float kc[L::RPT], gc[L::RPT], muc, kn[L::RPT], gn[L::RPT], mun;
            load_kgm<L, M, TIn>(p.f, bth_of(n * C), rg, kc, gc, muc);
            for (int tau = 0; tau < C; ++tau) {
                // loads before stores, unconditional, as in the elementwise rerun above
                load_kgm<L, M, TIn>(p.f, bth_of(n * C + (tau + 1 < C ? tau + 1 : tau)), rg, kn, gn, mun);
#pragma unroll
                for (int i = 0; i < L::RPT; ++i)
                    *reinterpret_cast<float4*>(rtok + static_cast<int64_t>(tau) * M * D + el(i)) = r[i];
                const float4 h = *reinterpret_cast<const float4*>(hbuf + tau * D + cg * 4);
                float c[L::RPT], beta[L::RPT], hh;
                fwd_token_h<L, LIN1>(z, r, kc, gc, muc, h, mode, c, beta, hh);
                float* rec = trec + static_cast<int64_t>(tau) * TR::SIZE;
                if (cg == 0) {
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i) {
                        rec[TR::C_OFF + rg + L::RG * i] = c[i];
                        rec[TR::B_OFF + rg + L::RG * i] = beta[i];
                    }
                }
                if (tid == 0) rec[TR::HH_OFF] = hh;
#pragma unroll
                for (int i = 0; i < L::RPT; ++i) {
                    kc[i] = kn[i];
                    gc[i] = gn[i];
                }
                muc = mun;
            }
        }
        __syncthreads();  // records visible to every thread

        // reverse walk, BT tokens per exchange over slots
        float4 dZ[L::RPT];
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) dZ[i] = f4(0.f);
        // (the staged split path has C >= 16 > BT: every batch is full, known at compile
        // time, so the batch is straight-line code)
        const int nb = STG ? BT : (C < BT ? C : BT);
        // the state after the chunk's last token is the next chunk's stored start;
        // the state after token tau - 1 is the state before token tau
        float4 rpost[L::RPT];
        if constexpr (PF_STATE) {
            const float* s1 = sck + static_cast<int64_t>(n + 1) * M * D;
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) rpost[i] = *reinterpret_cast<const float4*>(s1 + el(i));
        }
        // With DBUF, token tau's values live in rv[tau & 1] (the batch starts ub are
        // even, so tau & 1 == u & 1 is fixed in the unrolled batch): the next
        // token's loads go to the other buffer, and no copy of registers with loads
        // in flight forces a wait.  Otherwise rv[0] is the current token and rv[1]
        // the prefetched next one, copied over at the end of each token.
        RevIn<L::RPT> rv[2];
        // token tau's inputs and record: from LDS (split workgroups) or memory
        auto lrev = [&](RevIn<L::RPT>& x, int tau) __attribute__((always_inline)) {
            if constexpr (STG)
                load_rev_staged<L, ML, D, DYB>(x, p, srec, rtok + static_cast<int64_t>(tau) * M * D,
                                               bth_of(n * C + tau), tau, rgl, cg, el(0));
            else
                load_rev<L, M, D, TIn, PF_STATE, DYB>(x, p, trec, rtok, bth_of(n * C + tau), ch, tau, rg, cg, el(0));
        };
        if constexpr (PF_TOKEN) {
            // (static indices only: a computed one would put rv in scratch memory)
            if (DBUF && C > 1)
                lrev(rv[1], C - 1);
            else
                lrev(rv[0], C - 1);
        }
        for (int ub = C - nb; ub >= 0; ub -= nb) {
            float* rb = WB::RED2 ? red + (nred++ & 1) * (BT * L::NW * W) : red;
            float dcv[BT][L::RPT], kv[BT][L::RPT], dkin[BT][L::RPT];
            float dqv[STG ? BT : 1][L::RPT], dgv[STG ? BT : 1][L::RPT];  // (STG: this batch's dq, dgamma)
#pragma unroll
            for (int u = BT - 1; u >= 0; --u) {
                if (u < nb) {
                    const int tau = ub + u;
                    const int64_t bth = bth_of(n * C + tau);
                    if constexpr (PF_TOKEN) {
                        // unconditional (token 0 loads itself again): a load under a
                        // branch would be waited for where the branch joins
                        const int tp = tau > 0 ? tau - 1 : 0;
                        lrev(rv[DBUF ? (u + 1) & 1 : 1], tp);
                    } else {
                        load_rev<L, M, D, TIn, false, DYB>(rv[0], p, trec, rtok, bth, ch, tau, rg, cg, el(0));
                    }
                    const RevIn<L::RPT>& rc = rv[DBUF ? u & 1 : 0];
                    const TokenIn<L::RPT>& in = rc.in;
                    const float4 h = *reinterpret_cast<const float4*>(hbuf + tau * D + cg * 4);
                    const float hh = rc.hh;
                    const float4 dy = rc.dy;
                    float4 rp[L::RPT];
                    if constexpr (PF_STATE) {
#pragma unroll
                        for (int i = 0; i < L::RPT; ++i) rp[i] = rc.rp[i];
                    } else {
                        const float* rpre = rtok + static_cast<int64_t>(tau) * M * D;
                        const float* rnext = tau == C - 1 ? sck + static_cast<int64_t>(n + 1) * M * D
                                                          : rtok + static_cast<int64_t>(tau + 1) * M * D;
#pragma unroll
                        for (int i = 0; i < L::RPT; ++i) {
                            rp[i] = *reinterpret_cast<const float4*>(rpre + el(i));
                            rpost[i] = *reinterpret_cast<const float4*>(rnext + el(i));
                        }
                    }

                    // reductions over d: dq, dg, dkap (and, first linearisation, the
                    // adjoint of the chunk-start term's coefficient, de = z . D)
                    float dq[L::RPT], dg[L::RPT], dk2[L::RPT], de[L::RPT];
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i) {
                        dq[i] = dot4(rpost[i], dy);
                        dR[i] = fma4(in.q[i], dy, dR[i]);
                        dg[i] = dot4(rp[i], dR[i]);
                        dk2[i] = dot4(h, dR[i]);
                        de[i] = LIN1 ? dot4(z[i], dR[i]) : 0.f;
                    }
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i) {
                        dq[i] = group_sum<L::TPR>(dq[i]);
                        dg[i] = group_sum<L::TPR>(dg[i]);
                        dk2[i] = group_sum<L::TPR>(dk2[i]);
                    }
                    if constexpr (LIN1) {
#pragma unroll
                        for (int i = 0; i < L::RPT; ++i) de[i] = group_sum<L::TPR>(de[i]);
                    }

                    // scalar chain rule per slot
                    const float mu = in.mu;
                    float gate[L::RPT], dgam[L::RPT];
                    float4 hp = f4(0.f);
                    float4 sc = f4(0.f);  // (d|h|^2, dmu, dgamma summed over slots, 0)
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i) {
                        const float ci = rc.c[i];
                        const float bt = rc.beta[i];
                        const float coef = enc ? ci - in.k[i] : in.k[i];
                        const float a = in.g[i] * coef;
                        const float wraw = fmaf(-ci, ci, hh);
                        const float w = fmaxf(wraw, 0.f);
                        const float kap = -bt * a;
                        float dbeta, da, dmu_i, dci;
                        if constexpr (LIN1) {
                            // g = mu beta, e = beta a c (coefficient of z), kap = -beta a
                            gate[i] = bt * mu;
                            dbeta = fmaf(mu, dg[i], a * (ci * de[i] - dk2[i]));
                            da = bt * (ci * de[i] - dk2[i]);
                            dmu_i = bt * dg[i];
                            dci = bt * a * de[i];
                            dZ[i] = fma4(bt * a * ci, dR[i], dZ[i]);
                        } else {
                            // g = beta (mu + a c), kap = -beta a
                            const float num = fmaf(a, ci, mu);
                            gate[i] = bt * num;
                            dbeta = num * dg[i] - a * dk2[i];
                            da = bt * (ci * dg[i] - dk2[i]);
                            dmu_i = bt * dg[i];
                            dci = bt * a * dg[i];
                        }
                        const float tb = -0.5f * bt * bt * bt * dbeta;
                        dmu_i = fmaf(2.f * mu, tb, dmu_i);
                        da = fmaf(2.f * a * w, tb, da);
                        const float dw = a * a * tb;
                        float dhh_i = 0.f;
                        if (wraw > 0.f) {
                            dhh_i = dw;
                            dci = fmaf(-2.f * ci, dw, dci);
                        }
                        if (enc) {
                            dci = fmaf(in.g[i], da, dci);
                            dkin[u][i] = -in.g[i] * da;
                            dgam[i] = coef * da;
                        } else {
                            dkin[u][i] = in.g[i] * da;
                            dgam[i] = in.k[i] * da;
                        }
                        dcv[u][i] = dci;
                        kv[u][i] = in.k[i];
                        hp = fma4(kap, dR[i], fma4(dci, z[i], hp));
                        sc.x += dhh_i;
                        sc.y += dmu_i;
                        sc.z += dgam[i];
                    }
                    // this token's partial sums over the wave's slots, to LDS
                    hp.x = strided_sum<L::TPR>(hp.x);
                    hp.y = strided_sum<L::TPR>(hp.y);
                    hp.z = strided_sum<L::TPR>(hp.z);
                    hp.w = strided_sum<L::TPR>(hp.w);
                    sc.x = strided_sum<L::TPR>(sc.x);
                    sc.y = strided_sum<L::TPR>(sc.y);
                    sc.z = strided_sum<L::TPR>(sc.z);
                    if constexpr (STG) {
                        // every row group holds the same sums: all lanes write (the same values
                        // to the same addresses), so the batch stays straight-line code
                        *reinterpret_cast<float4*>(rb + (u * L::NW + wave) * W + cg * 4) = hp;
                        *reinterpret_cast<float4*>(rb + (u * L::NW + wave) * W + D) = sc;
                    } else {
                        if (lane < L::TPR) *reinterpret_cast<float4*>(rb + (u * L::NW + wave) * W + cg * 4) = hp;
                        if (lane == 0) *reinterpret_cast<float4*>(rb + (u * L::NW + wave) * W + D) = sc;
                    }
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i) {
                        dR[i] = gate[i] * dR[i];
                        if constexpr (PF_STATE) rpost[i] = rp[i];
                    }
                    if constexpr (PF_TOKEN && !DBUF) rv[0] = rv[1];
                    if constexpr (STG) {
                        // stored after the batch (no branch in the token's code)
#pragma unroll
                        for (int i = 0; i < L::RPT; ++i) {
                            dqv[u][i] = dq[i];
                            dgv[u][i] = dgam[i];
                        }
                    } else if (cg == 0) {
#pragma unroll
                        for (int i = 0; i < L::RPT; ++i) {
                            const int64_t o = bth * M + rg + L::RG * i;
                            p.dq[o] = dq[i];
                            if (p.f.gamma_per_slot) p.dgamma[o] = dgam[i];
                        }
                    }
                }
            }
            __syncthreads();  // the batch's partial sums visible
            // the sums over waves, one float4 of the batch per thread
            const bool mine = tid < nb * (D / 4 + 1);
            const int xu = tid / (D / 4 + 1), xc4 = tid % (D / 4 + 1);
            float4 acc = f4(0.f);
            if (mine) {
                acc = *reinterpret_cast<const float4*>(rb + (xu * L::NW) * W + xc4 * 4);
#pragma unroll
                for (int w = 1; w < L::NW; ++w) acc = acc + *reinterpret_cast<const float4*>(rb + (xu * L::NW + w) * W + xc4 * 4);
            }
            if constexpr (P > 1) {
                // The other workgroups' sums of this batch (over their rows): publish
                // this one's, wait for theirs, add all in workgroup order (the same
                // operations in every workgroup).  Parts alternate between two
                // buffers by batch parity: a buffer is rewritten two batches later,
                // after every workgroup has published the batch in between, which
                // each does only after reading this one.
                constexpr int XW = 8 * W;  // floats per part (batches of at most 8 tokens)
                static_assert(BT <= 8, "hand-off part size");
                float* xb = p.xbuf + (static_cast<int64_t>(bh) * 2 + (nbatch & 1)) * P * XW;
                const __amdgpu_buffer_rsrc_t xr = xrsrc(xb, static_cast<uint32_t>(P * XW * sizeof(float)));
                const uint32_t off = static_cast<uint32_t>(xu * W + xc4 * 4) * 4;
                if (mine)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(bwd_u32x4, acc), xr,
                                                           static_cast<uint32_t>(pidx * XW) * 4 + off, 0, XCPOL_SC1);
                asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this thread's part store has retired
                __syncthreads();  // ... and every thread's
                if (tid == 0)
                    __hip_atomic_store(p.xflags + (bh * P + pidx) * XFLAG_STRIDE, nbatch + 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                // thread q polls workgroup q's counter (all P at once, one round trip when they are set)
                if (tid < P && tid != pidx && !xbroken) {
                    const int* f = p.xflags + (bh * P + tid) * XFLAG_STRIDE;
                    int n = 0;
                    while (__hip_atomic_load(const_cast<int*>(f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= nbatch) {
                        if (++n >= XSPIN) {
                            xbroken = true;
                            break;
                        }
                    }
                }
                __syncthreads();  // the other parts are published
                asm volatile("" ::: "memory");  // the reads below stay after the barrier
                if (mine) {
                    float4 part[P];
#pragma unroll
                    for (int q = 0; q < P; ++q)
                        part[q] = q == pidx ? acc
                                            : __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                             xr, static_cast<uint32_t>(q * XW) * 4 + off,
                                                                             0, XCPOL_SC1));
                    acc = part[0];
#pragma unroll
                    for (int q = 1; q < P; ++q) acc = acc + part[q];
                }
                ++nbatch;
            }
            if (mine) *reinterpret_cast<float4*>(tot + xu * W + xc4 * 4) = acc;
            __syncthreads();  // the batch's sums visible
#pragma unroll
            for (int u = 0; u < BT; ++u) {
                if (u < nb) {
                    const int tau = ub + u;
                    const int64_t bth = bth_of(n * C + tau);
                    const float4 hsum = *reinterpret_cast<const float4*>(tot + u * W + cg * 4);
                    const float4 ssum = *reinterpret_cast<const float4*>(tot + u * W + D);
                    const float4 h = *reinterpret_cast<const float4*>(hbuf + tau * D + cg * 4);
                    const float4 dh = fma4(2.f * ssum.x, h, hsum);
                    float dkz[L::RPT] = {};
#pragma unroll
                    for (int i = 0; i < L::RPT; ++i) {
                        dZ[i] = fma4(dcv[u][i], h, dZ[i]);
                        if (mode == 0) {
                            dZ[i] = fma4(kv[u][i], dh, dZ[i]);
                            dkz[i] = dot4(z[i], dh);
                        }
                    }
                    if (mode == 0) {
#pragma unroll
                        for (int i = 0; i < L::RPT; ++i) dkz[i] = group_sum<L::TPR>(dkz[i]);
                    }
                    if (cg == 0) {
#pragma unroll
                        for (int i = 0; i < L::RPT; ++i) p.dk[bth * M + rg + L::RG * i] = dkin[u][i] + dkz[i];
                        if constexpr (STG) {
#pragma unroll
                            for (int i = 0; i < L::RPT; ++i) {
                                const int64_t o = bth * M + rg + L::RG * i;
                                p.dq[o] = dqv[u][i];
                                if (p.f.gamma_per_slot) p.dgamma[o] = dgv[u][i];
                            }
                        }
                    }
                    if (tid == 0 && pidx == 0) {
                        p.dmu[bth] = ssum.y;
                        if (!p.f.gamma_per_slot) p.dgamma[bth] = ssum.z;
                    }
                    if (rg == 0) *reinterpret_cast<float4*>(p.dv + bth * D + cg * 4) = mode == 2 ? dh : f4(0.f) - dh;
                }
            }
        }

        // gradient of Z (running path + frozen uses) back through the projection
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) {
            const float4 dz = dR[i] + dZ[i];
            const float pz = group_sum<L::TPR>(dot4(z[i], dz));
            dR[i] = inv[i] * fma4(-pz, z[i], dz);
        }
    }

    float* dsi = p.dstate_in + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) *reinterpret_cast<float4*>(dsi + el(i)) = dR[i];
}

template <int N>
__global__ void osr_bwd_fill_ints(int* x, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) x[i] = N;
}

template <int M, int D, int NT, typename TIn, int P>
static void launch_bwd_dy(const BwdParams& p, dim3 grid, size_t lds, hipStream_t st) {
    if (p.f.lin1) {
        if (p.dy_bf16)
            hipLaunchKernelGGL((osr_bwd_kernel<M, D, NT, TIn, true, true, P>), grid, dim3(NT), lds, st, p);
        else
            hipLaunchKernelGGL((osr_bwd_kernel<M, D, NT, TIn, true, false, P>), grid, dim3(NT), lds, st, p);
    } else {
        if (p.dy_bf16)
            hipLaunchKernelGGL((osr_bwd_kernel<M, D, NT, TIn, false, true, P>), grid, dim3(NT), lds, st, p);
        else
            hipLaunchKernelGGL((osr_bwd_kernel<M, D, NT, TIn, false, false, P>), grid, dim3(NT), lds, st, p);
    }
}

// Launch for one slot count M, width D and P workgroups per sequence (M / P
// slot rows each; P > 1 only with bf16 inputs and the state-passing kernel's
// arrays, which the host ensures).
template <int M, int D, int P>
static int launch_bwd_mdp(const BwdParams& p, bool in_bf16, hipStream_t st) {
    constexpr int TPR = D / 4;
    constexpr int NT = ((M / P) * TPR < 512) ? (M / P) * TPR : 512;
    const dim3 grid(static_cast<unsigned>(p.f.B) * static_cast<unsigned>(p.f.H) * P);
    using L = ValuLayout<M / P, D, NT>;
    using WB = WalkBatch<M, D, NT, P>;
    constexpr size_t static_lds = (WB::RED + WB::TOT) * sizeof(float);  // red, tot
    const size_t h_lds = static_cast<size_t>(p.f.chunk) * D * sizeof(float);      // the chunk's h
    const size_t gk_lds = static_cast<size_t>(p.f.lin1 ? 3 : 2) * M * p.f.chunk * sizeof(float);
    // the chunk's gates from the state-passing kernel, staged in LDS where it fits
    // split workgroups: the chunk's records of their rows (StagedRec)
    constexpr bool STG = P > 1 && L::RPT <= 2 && M / P <= 32;
    const size_t rec_lds = STG ? static_cast<size_t>(StagedRec<M / P, D>::floats(p.f.chunk)) * sizeof(float) : 0;
    BwdParams q = p;
    q.stage_gk = p.chain_c != nullptr && static_lds + h_lds + rec_lds + gk_lds <= 128 * 1024;
    const size_t lds = h_lds + (q.stage_gk ? gk_lds : 0) + rec_lds;
    if (static_lds + lds > 160 * 1024) return -3;  // (the split policy never picks such a P)
    if constexpr (P > 1) {
        // progress counters to zero (they count the batches of this call)
        const int nflags = p.f.B * p.f.H * P * XFLAG_STRIDE;
        hipLaunchKernelGGL(osr_bwd_fill_ints<0>, dim3((nflags + 255) / 256), dim3(256), 0, st, p.xflags, nflags);
        launch_bwd_dy<M, D, NT, uint16_t, P>(q, grid, lds, st);
    } else {
        // the first linearisation is its own instantiation, so the default carries none of its work;
        // so is a bf16 dy (its loads then need no branch)
        if (in_bf16)
            launch_bwd_dy<M, D, NT, uint16_t, 1>(q, grid, lds, st);
        else
            launch_bwd_dy<M, D, NT, float, 1>(q, grid, lds, st);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int M, int D>
static int launch_bwd_md(const BwdParams& p, bool in_bf16, hipStream_t st) {
    if (p.split_p > 1 && (!in_bf16 || p.chain_c == nullptr || p.xbuf == nullptr)) return -3;
    switch (p.split_p) {
        case 1: return launch_bwd_mdp<M, D, 1>(p, in_bf16, st);
        case 2:
            if constexpr (M / 2 >= 16) return launch_bwd_mdp<M, D, 2>(p, in_bf16, st);
            return -3;
        case 4:
            if constexpr (M / 4 >= 16) return launch_bwd_mdp<M, D, 4>(p, in_bf16, st);
            return -3;
        case 8:
            if constexpr (M / 8 >= 16) return launch_bwd_mdp<M, D, 8>(p, in_bf16, st);
            return -3;
        default: return -3;
    }
}

template <int M>
int launch_bwd_m(int d, const BwdParams& p, bool in_bf16, hipStream_t st) {
    switch (d) {
        case 16: return launch_bwd_md<M, 16>(p, in_bf16, st);
        case 32: return launch_bwd_md<M, 32>(p, in_bf16, st);
        case 64: return launch_bwd_md<M, 64>(p, in_bf16, st);
        case 128: return launch_bwd_md<M, 128>(p, in_bf16, st);
        default: return -3;
    }
}

}  // namespace osr
