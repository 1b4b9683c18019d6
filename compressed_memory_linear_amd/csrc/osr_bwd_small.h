// osr_bwd_small.h -- reverse walk of the backward at small chunks (C = 1, 2, 4, 8
// after the token loop, 16 after the matrix-core state passing).
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646), section "Parallel and Hardware Efficient Form", eq.
// recurrence_linear2 (the default linearisation).  The vector-Jacobian product
// is that of the general walk (osr_bwd_kernel.h states the per-token reverse);
// this kernel is its form for chunks short enough that the state before and
// after every token of a chunk stays in registers.
//
// Phase 1 is the small-chunk token loop of the forward (osr_valu.hip), which
// leaves every chunk-start state (before projection) in the workspace, in the
// layout of the general walk, and for the decoding objective every token's h.
// This kernel then walks the chunks backwards, one workgroup per (b,h), in
// the token loop's thread layout:
//   - a chunk's inputs (h, dy, k, q, gamma, mu of its C tokens) are staged in
//     LDS by all threads together, each thread's loads issued one chunk ahead
//     and converted to fp32 only when written to LDS; the chunk-start state
//     is read one chunk ahead the same way;
//   - c and |h|^2 of the chunk's tokens depend only on the projected start
//     state z and on h, so all C (RPT + 1) row sums run together; the forward
//     is rerun elementwise from z;
//   - in the reverse the adjoint of the state is only scaled by the gate and
//     takes q dy per token, so no token's row sums (dq, dg, dkap) feed the
//     next token's: they follow one another without waiting, and the partial
//     sums over slots of all C tokens go through one LDS exchange;
//   - two barriers per chunk: one publishes the partial sums, the other the
//     sums over waves together with the next chunk's staged inputs.
// The walk is bound by VALU issue on the B*H compute units that hold a
// sequence.  With P = 2 or 4 the slot rows of a sequence split over P
// workgroups (M / P rows each, 1/P of the instructions per chunk); every
// row-local step is unchanged, and the chunk's sums over slots, the only step
// that crosses rows, go from workgroup to workgroup as tagged 64-bit pairs
// (below); each adds all parts in workgroup order, so all hold the same sums.
#pragma once

#include <type_traits>

#include "osr_bwd_kernel.h"
#include "osr_launch.h"
#include "osr_valu.h"

namespace osr {

// Threads per workgroup of the walk with the rows split over P workgroups.
template <int M, int D, int P>
constexpr int bwd_small_threads() {
    return tokenloop_threads<M / P, D>();
}

// Whether the walk runs on P workgroups of M / P rows each: 16 rows or more
// (P > 1), at most 2 slot rows per thread (the chunk's states in registers), and
// the threads to stage a chunk's inputs and hold its sums, one unit of each kind
// per thread.
template <int M, int D, int C, int P>
constexpr bool bwd_small_split_ok() {
    if constexpr (M / P < 16 && P > 1) {
        return false;
    } else {
        constexpr int NT = bwd_small_threads<M, D, P>();
        constexpr int RPT = ValuLayout<M / P, D, NT>::RPT;
        return RPT <= 2 && C * RPT <= 16 && C * (M / 4) <= NT && C * (D / 4 + 1) <= NT;
    }
}

// Whether the small-chunk walk is built for (M, D, C): at C <= 8 within the
// forward token loop's exchange batch (its phase 1; at C = 16 the matrix-core
// state passing is phase 1), and some P in {1, 2, 4} that bwd_small_split_ok
// allows.
template <int M, int D>
constexpr bool bwd_small_fits(int C) {
    using L = ValuLayout<M, D, tokenloop_threads<M, D>()>;
    if (!(((C == 1 || C == 2 || C == 4 || C == 8) && C <= TokBatch<L>::BT) || C == 16)) return false;
    switch (C) {
        case 1: return bwd_small_split_ok<M, D, 1, 1>() || bwd_small_split_ok<M, D, 1, 2>() || bwd_small_split_ok<M, D, 1, 4>();
        case 2: return bwd_small_split_ok<M, D, 2, 1>() || bwd_small_split_ok<M, D, 2, 2>() || bwd_small_split_ok<M, D, 2, 4>();
        case 4: return bwd_small_split_ok<M, D, 4, 1>() || bwd_small_split_ok<M, D, 4, 2>() || bwd_small_split_ok<M, D, 4, 4>();
        case 8: return bwd_small_split_ok<M, D, 8, 1>() || bwd_small_split_ok<M, D, 8, 2>() || bwd_small_split_ok<M, D, 8, 4>();
        default: return bwd_small_split_ok<M, D, 16, 1>() || bwd_small_split_ok<M, D, 16, 2>() || bwd_small_split_ok<M, D, 16, 4>();
    }
}

// Four consecutive elements loaded without conversion (the conversion, and so
// the wait for the load, happens where the value is used).
template <typename T>
struct Raw4;
template <>
struct Raw4<float> {
    using type = float4;
    __device__ static type load(const float* p, int64_t i) { return *reinterpret_cast<const float4*>(p + i); }
    __device__ static float4 cvt(type v) { return v; }
};
template <>
struct Raw4<uint16_t> {
    using type = uint2;
    __device__ static type load(const uint16_t* p, int64_t i) { return *reinterpret_cast<const uint2*>(p + i); }
    __device__ static float4 cvt(type u) {
        return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u), __uint_as_float(u.y << 16),
                           __uint_as_float(u.y & 0xFFFF0000u));
    }
};
template <typename T>
struct Raw1;
template <>
struct Raw1<float> {
    using type = float;
    __device__ static type load(const float* p, int64_t i) { return p[i]; }
    __device__ static float cvt(type v) { return v; }
};
template <>
struct Raw1<uint16_t> {
    using type = uint16_t;
    __device__ static type load(const uint16_t* p, int64_t i) { return p[i]; }
    __device__ static float cvt(type v) { return bf16_bits_to_f32(v); }
};

// A chunk's staged inputs in LDS (floats): h and dy [C][D], k, q and a
// per-slot gamma [C][M], mu and a per-token gamma [C].
template <int M, int D, int C>
struct SmallStage {
    static constexpr int H = 0, DY = C * D, K = 2 * C * D, Q = K + C * M, G = Q + C * M, MU = G + C * M, GT = MU + C;
    static constexpr int SIZE = (GT + C + 3) / 4 * 4;
};

// DEC: decoding objective (h = sum_i k_i z_i - v, from the phase-1 records:
// the token loop's [T][D] rows, or with CH the state-passing kernel's per-chunk
// fragments); otherwise h = -v (similarity) or v (encoding layer).  DYB: dy in
// bf16.  LIN1: the first chunk linearisation (eq. recurrence_linear1: gate
// mu beta, and the term beta a c z on the chunk-start slot), whose reverse takes
// one more row sum per token, de = z . D, and gives the term's share of dZ.
template <int M, int D, int NT, int C, typename TIn, bool DYB, bool DEC, int P, bool CH = false, bool LIN1 = false>
__global__ __launch_bounds__(NT) void osr_bwd_small_kernel(BwdParams p) {
    static_assert(bwd_small_split_ok<M, D, C, P>(), "rows, registers and threads of the split");
    using L = ValuLayout<M / P, D, NT>;
    using SG = SmallStage<M, D, C>;
    using DYT = typename std::conditional<DYB, uint16_t, float>::type;
    using HT = typename std::conditional<DEC, float, TIn>::type;
    constexpr int RPT = L::RPT, Q = D / 4, MQ = M / 4, W = D + 4, NW = L::NW;
    static_assert(RPT <= 2, "the chunk's states in registers");
    static_assert(C * Q <= NT && C * MQ <= NT && 2 * C <= NT, "one staged unit of each kind per thread");
    static_assert(C * (Q + 1) <= NT, "one float4 of the chunk's sums per thread");
    __shared__ __attribute__((aligned(16))) float stg[2 * SG::SIZE];  // staged inputs, by chunk parity
    __shared__ __attribute__((aligned(16))) float red[C * NW * W];    // partial sums over each wave's slots
    __shared__ __attribute__((aligned(16))) float tot[C * W];         // the chunk's sums over slots

    const int bh = P > 1 ? blockIdx.x / P : blockIdx.x;
    const int pidx = P > 1 ? blockIdx.x % P : 0;  // this workgroup's rows: [pidx M/P, (pidx + 1) M/P)
    const int b = bh / p.f.H, hd = bh % p.f.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // rg: the (global) slot row of this thread's first row
    const int cg = tid % L::TPR, rg = pidx * (M / P) + tid / L::TPR;
    int nxch = 0;          // chunks exchanged with the other workgroups (P > 1)
    bool xbroken = false;  // a wait for them gave up (then the results are wrong, but every wave ends)
    const int T = p.f.T, NC = T / C;
    const bool enc = p.f.mode == 2;
    const bool gps = p.f.gamma_per_slot != 0;
    auto bth_of = [&](int t) { return (static_cast<int64_t>(b) * T + t) * p.f.H + hd; };
    auto el = [&](int i) { return (rg + L::RG * i) * D + cg * 4; };
    float* const sck = p.ws + static_cast<int64_t>(bh) * bwd_floats_per_bh<M, D>(T, C);  // [NC+1][M][D]
    const float* const hrec = DEC && !CH ? p.f.hrec + static_cast<int64_t>(bh) * T * D : nullptr;

    // ---- staging: this thread's unit of each kind (indices clamped; only the
    // threads inside a kind's range write it) ----
    const TIn* kp = static_cast<const TIn*>(p.f.k);
    const TIn* qp = static_cast<const TIn*>(p.f.q);
    const TIn* gp = static_cast<const TIn*>(p.f.gamma);
    const TIn* vp = static_cast<const TIn*>(p.f.v);
    const TIn* mp = static_cast<const TIn*>(p.f.mu);
    const DYT* dyp = static_cast<const DYT*>(p.dy);
    const int jq = tid < C * Q ? tid : C * Q - 1, uq = jq / Q, cq = jq % Q;      // h, dy
    const int jm = tid < C * MQ ? tid : C * MQ - 1, um = jm / MQ, rm = jm % MQ;  // k, q, gamma
    const int us = tid % C;                                                     // mu, per-token gamma
    // (per-token gamma: no per-slot array, the k unit is loaded again in its place;
    // the scalar unit reads gamma for threads C .. 2C - 1 then)
    const TIn* gsl = gps ? gp : kp;
    const TIn* ssrc = (!gps && tid >= C) ? gp : mp;
    struct Pre {
        typename Raw4<HT>::type h;
        typename Raw4<DYT>::type dy;
        typename Raw4<TIn>::type k, q, g;
        typename Raw1<TIn>::type s;
        float4 st[RPT];
    };
    auto issue = [&](Pre& x, int n) __attribute__((always_inline)) {
        const int64_t bq = bth_of(n * C + uq), bm = bth_of(n * C + um);
        if constexpr (DEC && CH) {
            // lane (lg, lc) of the fragment for column block jb and token tile tb holds
            // h[16 tb + 4 lg + r][16 jb + lc]: the 4 columns of a unit are 4 floats apart
            const float* hs = p.chain_h + (static_cast<int64_t>(bh) * NC + n) * D * C +
                              ((static_cast<int64_t>(cq >> 2) * (C >> 4) + (uq >> 4)) * 64 + ((uq & 15) >> 2) * 16 +
                               (cq & 3) * 4) * 4 + (uq & 3);
            x.h = make_float4(hs[0], hs[4], hs[8], hs[12]);
        } else if constexpr (DEC)
            x.h = Raw4<float>::load(hrec, static_cast<int64_t>(n * C + uq) * D + cq * 4);
        else
            x.h = Raw4<TIn>::load(vp, bq * D + cq * 4);
        x.dy = Raw4<DYT>::load(dyp, bq * D + cq * 4);
        x.k = Raw4<TIn>::load(kp, bm * M + rm * 4);
        x.q = Raw4<TIn>::load(qp, bm * M + rm * 4);
        x.g = Raw4<TIn>::load(gsl, bm * M + rm * 4);
        x.s = Raw1<TIn>::load(ssrc, bth_of(n * C + us));
#pragma unroll
        for (int i = 0; i < RPT; ++i) x.st[i] = *reinterpret_cast<const float4*>(sck + static_cast<int64_t>(n) * M * D + el(i));
    };
    const float hsgn = p.f.mode == 2 ? 1.f : -1.f;
    auto commit = [&](const Pre& x, float* sb) __attribute__((always_inline)) {
        if (tid < C * Q) {
            const float4 hv = Raw4<HT>::cvt(x.h);
            *reinterpret_cast<float4*>(sb + SG::H + uq * D + cq * 4) = DEC ? hv : hsgn * hv;
            *reinterpret_cast<float4*>(sb + SG::DY + uq * D + cq * 4) = Raw4<DYT>::cvt(x.dy);
        }
        if (tid < C * MQ) {
            *reinterpret_cast<float4*>(sb + SG::K + um * M + rm * 4) = Raw4<TIn>::cvt(x.k);
            *reinterpret_cast<float4*>(sb + SG::Q + um * M + rm * 4) = Raw4<TIn>::cvt(x.q);
            *reinterpret_cast<float4*>(sb + SG::G + um * M + rm * 4) = Raw4<TIn>::cvt(x.g);
        }
        if (tid < 2 * C) sb[SG::MU + tid] = Raw1<TIn>::cvt(x.s);  // (MU, then GT)
    };

    // ---- the returned state is the end state projected: its backward ----
    float4 dR[RPT];
    {
        const float* dso = p.dstate_out + static_cast<int64_t>(bh) * M * D;
        float4 r[RPT], o[RPT];
        float n2[RPT], pr[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            r[i] = *reinterpret_cast<const float4*>(sck + static_cast<int64_t>(NC) * M * D + el(i));
            dR[i] = *reinterpret_cast<const float4*>(dso + el(i));
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) n2[i] = group_sum<L::TPR>(dot4(r[i], r[i]));
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            o[i] = rsqrtf(n2[i]) * r[i];
            pr[i] = group_sum<L::TPR>(dot4(o[i], dR[i]));
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) dR[i] = rsqrtf(n2[i]) * fma4(-pr[i], o[i], dR[i]);
    }

    // ---- one chunk's steps ----
    // A chunk prepared for its reverse: the projected start state, c and |h|^2 of
    // its tokens, beta, and the state before every token and after the last
    // (h too at C <= 4; at C = 8 it is read from LDS where used: held, it spilled).
    constexpr int HC = C > 4 ? 1 : C;
    struct Prep {
        float inv[RPT];
        float4 z[RPT];
        float cc[C][RPT + 1];
        float beta[C][RPT];
        float4 rs[C + 1][RPT];
        float4 h[HC];
    };
    auto stage_of = [&](int n) { return stg + (n & 1) * SG::SIZE; };
    auto hat = [&](const Prep& x, const float* sb, int u) __attribute__((always_inline)) {
        if constexpr (C > 4)
            return *reinterpret_cast<const float4*>(sb + SG::H + u * D + cg * 4);
        else
            return x.h[u];
    };
    // c and |h|^2 of every token depend only on z and h: all C (RPT + 1) row sums
    // together; then the forward again, elementwise
    auto prep = [&](Prep& x, int n, const float4 (&s)[RPT]) __attribute__((always_inline)) {
        const float* sb = stage_of(n);
        float n2[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) n2[i] = group_sum<L::TPR>(dot4(s[i], s[i]));
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            x.inv[i] = rsqrtf(n2[i]);
            x.z[i] = x.inv[i] * s[i];
        }
        float4 h[C];
#pragma unroll
        for (int u = 0; u < C; ++u) h[u] = *reinterpret_cast<const float4*>(sb + SG::H + u * D + cg * 4);
#pragma unroll
        for (int u = 0; u < C; ++u) {
#pragma unroll
            for (int i = 0; i < RPT; ++i) x.cc[u][i] = dot4(x.z[i], h[u]);
            x.cc[u][RPT] = dot4(h[u], h[u]);
        }
#pragma unroll
        for (int u = 0; u < C; ++u)
#pragma unroll
            for (int i = 0; i <= RPT; ++i) x.cc[u][i] = group_sum<L::TPR>(x.cc[u][i]);
#pragma unroll
        for (int i = 0; i < RPT; ++i) x.rs[0][i] = x.z[i];
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const float mu = sb[SG::MU + u], hh = x.cc[u][RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg + L::RG * i;
                const float k = sb[SG::K + u * M + row];
                const float g = sb[gps ? SG::G + u * M + row : SG::GT + u];
                const float ci = x.cc[u][i];
                const float a = g * (enc ? ci - k : k);
                const float w = fmaxf(fmaf(-ci, ci, hh), 0.f);
                const float bt = rsqrtf(fmaf(mu, mu, a * a * w));
                x.beta[u][i] = bt;
                if constexpr (LIN1)
                    x.rs[u + 1][i] = fma4(bt * mu, x.rs[u][i], fma4(bt * a * ci, x.z[i], (-bt * a) * h[u]));
                else
                    x.rs[u + 1][i] = fma4(bt * fmaf(a, ci, mu), x.rs[u][i], (-bt * a) * h[u]);
            }
        }
        if constexpr (C <= 4) {
#pragma unroll
            for (int u = 0; u < C; ++u) x.h[u] = h[u];
        }
    };
    // the chunk's tokens in reverse: dq, per-slot dgamma; per token the partial
    // sums over the wave's slots (dh's terms, d|h|^2, dmu, per-token dgamma) to red
    // (dZl: the first linearisation's share of dZ, from the state's adjoint per token)
    auto reverse = [&](const Prep& x, int n, float (&dcv)[C][RPT], float (&dkin)[C][RPT], float4 (&dZl)[RPT])
                       __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < RPT; ++i) dZl[i] = f4(0.f);
        const float* sb = stage_of(n);
#pragma unroll
        for (int u = C - 1; u >= 0; --u) {
            const int64_t bth = bth_of(n * C + u);
            const float4 dy = *reinterpret_cast<const float4*>(sb + SG::DY + u * D + cg * 4);
            const float4 hu = hat(x, sb, u);
            const float mu = sb[SG::MU + u], hh = x.cc[u][RPT];
            float qv[RPT], kv[RPT], gv[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int row = rg + L::RG * i;
                qv[i] = sb[SG::Q + u * M + row];
                kv[i] = sb[SG::K + u * M + row];
                gv[i] = sb[gps ? SG::G + u * M + row : SG::GT + u];
            }
            float dq[RPT], dg[RPT], dk2[RPT], de[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                dq[i] = dot4(x.rs[u + 1][i], dy);
                dR[i] = fma4(qv[i], dy, dR[i]);
                dg[i] = dot4(x.rs[u][i], dR[i]);
                dk2[i] = dot4(hu, dR[i]);
                de[i] = LIN1 ? dot4(x.z[i], dR[i]) : 0.f;
            }
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                dq[i] = group_sum<L::TPR>(dq[i]);
                dg[i] = group_sum<L::TPR>(dg[i]);
                dk2[i] = group_sum<L::TPR>(dk2[i]);
                if constexpr (LIN1) de[i] = group_sum<L::TPR>(de[i]);
            }
            // scalar chain rule per slot: g = beta (mu + a c), kap = -beta a,
            // beta = (mu^2 + a^2 w)^(-1/2), w = max(|h|^2 - c^2, 0)
            float gate[RPT], dgam[RPT];
            float4 hp = f4(0.f);
            float4 sc = f4(0.f);  // (d|h|^2, dmu, dgamma summed over slots, 0)
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const float ci = x.cc[u][i], bt = x.beta[u][i];
                const float coef = enc ? ci - kv[i] : kv[i];
                const float a = gv[i] * coef;
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
                    dZl[i] = fma4(bt * a * ci, dR[i], dZl[i]);
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
                    dci = fmaf(gv[i], da, dci);
                    dkin[u][i] = -gv[i] * da;
                } else {
                    dkin[u][i] = gv[i] * da;
                }
                dgam[i] = coef * da;
                dcv[u][i] = dci;
                hp = fma4(kap, dR[i], fma4(dci, x.z[i], hp));
                sc.x += dhh_i;
                sc.y += dmu_i;
                sc.z += dgam[i];
            }
            hp.x = strided_sum<L::TPR>(hp.x);
            hp.y = strided_sum<L::TPR>(hp.y);
            hp.z = strided_sum<L::TPR>(hp.z);
            hp.w = strided_sum<L::TPR>(hp.w);
            sc.x = strided_sum<L::TPR>(sc.x);
            sc.y = strided_sum<L::TPR>(sc.y);
            sc.z = strided_sum<L::TPR>(sc.z);
            if (lane < L::TPR) *reinterpret_cast<float4*>(red + (u * NW + wave) * W + cg * 4) = hp;
            if (lane == 0) *reinterpret_cast<float4*>(red + (u * NW + wave) * W + D) = sc;
#pragma unroll
            for (int i = 0; i < RPT; ++i) dR[i] = gate[i] * dR[i];
            if (cg == 0) {
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    const int64_t o = bth * M + rg + L::RG * i;
                    p.dq[o] = dq[i];
                    if (gps) p.dgamma[o] = dgam[i];
                }
            }
        }
    };
    // the sums over waves, one float4 of the chunk per thread (mine)
    const bool mine = tid < C * (Q + 1);
    const int xu = tid / (Q + 1), xc4 = tid % (Q + 1);
    auto wave_sums = [&]() __attribute__((always_inline)) {
        float4 acc = f4(0.f);
        if (mine) {
            acc = *reinterpret_cast<const float4*>(red + (xu * NW) * W + xc4 * 4);
#pragma unroll
            for (int w = 1; w < NW; ++w) acc = acc + *reinterpret_cast<const float4*>(red + (xu * NW + w) * W + xc4 * 4);
        }
        return acc;
    };
    // gradients that take the sums over slots (tot); the gradient of Z back through
    // the projection, which leaves dR the gradient of the chunk before's end state
    auto finish = [&](const Prep& x, int n, const float (&dcv)[C][RPT], const float (&dkin)[C][RPT],
                      const float4 (&dZl)[RPT]) __attribute__((always_inline)) {
        const float* sb = stage_of(n);
        float4 dZ[RPT];
#pragma unroll
        for (int i = 0; i < RPT; ++i) dZ[i] = dZl[i];
#pragma unroll
        for (int u = 0; u < C; ++u) {
            const int64_t bth = bth_of(n * C + u);
            const float4 hsum = *reinterpret_cast<const float4*>(tot + u * W + cg * 4);
            const float4 ssum = *reinterpret_cast<const float4*>(tot + u * W + D);
            const float4 hu = hat(x, sb, u);
            const float4 dh = fma4(2.f * ssum.x, hu, hsum);
            float dkz[RPT] = {};
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                dZ[i] = fma4(dcv[u][i], hu, dZ[i]);
                if constexpr (DEC) {
                    dZ[i] = fma4(sb[SG::K + u * M + rg + L::RG * i], dh, dZ[i]);
                    dkz[i] = dot4(x.z[i], dh);
                }
            }
            if constexpr (DEC) {
#pragma unroll
                for (int i = 0; i < RPT; ++i) dkz[i] = group_sum<L::TPR>(dkz[i]);
            }
            if (cg == 0) {
#pragma unroll
                for (int i = 0; i < RPT; ++i) p.dk[bth * M + rg + L::RG * i] = dkin[u][i] + dkz[i];
            }
            // (every workgroup of a sequence holds the same sums: the first writes them)
            if (tid == 0 && pidx == 0) {
                p.dmu[bth] = ssum.y;
                if (!gps) p.dgamma[bth] = ssum.z;
            }
            if (rg == 0) *reinterpret_cast<float4*>(p.dv + bth * D + cg * 4) = enc ? dh : f4(0.f) - dh;
        }
#pragma unroll
        for (int i = 0; i < RPT; ++i) {
            const float4 dz = dR[i] + dZ[i];
            const float pz = group_sum<L::TPR>(dot4(x.z[i], dz));
            dR[i] = x.inv[i] * fma4(-pz, x.z[i], dz);
        }
    };

    Pre pre;
    issue(pre, NC - 1);
    commit(pre, stage_of(NC - 1));
    float4 scur[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) scur[i] = pre.st[i];
    __syncthreads();  // the last chunk's inputs visible
    issue(pre, NC > 1 ? NC - 2 : 0);

    // Split rows (P > 1): the chunk's sums over slots need the other workgroups'
    // parts.  Each value goes with the chunk's tag (nxch + 1) as one 64-bit pair,
    // written and read with agent-scope atomics, so a pair is seen whole or not at
    // all: publish writes this workgroup's pairs, await_part polls each other
    // workgroup's pairs of the thread's own float4 until all carry the tag (no
    // store-retire wait, barrier or counter on the way) and adds all parts in
    // workgroup order, so every workgroup holds the same sums.  Parts alternate
    // between two buffers by chunk parity: a workgroup rewrites a buffer two
    // chunks later, after every other one has published the chunk in between,
    // which each does only after reading this one.  The buffers are zeroed before
    // each call (tags start at 1).
    constexpr int XW = (C > 8 ? C : 8) * W;  // pairs per part
    auto xpart = [&](int q) __attribute__((always_inline)) {
        return reinterpret_cast<uint64_t*>(p.xbuf) + ((static_cast<int64_t>(bh) * 2 + (nxch & 1)) * P + q) * XW +
               xu * W + xc4 * 4;
    };
    auto publish = [&](float4 acc) __attribute__((always_inline)) {
        if (mine) {
            uint64_t* dst = xpart(pidx);
            const uint64_t tag = static_cast<uint64_t>(nxch + 1) << 32;
            __hip_atomic_store(dst + 0, tag | __float_as_uint(acc.x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(dst + 1, tag | __float_as_uint(acc.y), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(dst + 2, tag | __float_as_uint(acc.z), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(dst + 3, tag | __float_as_uint(acc.w), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    };
    auto await_part = [&](float4 acc) __attribute__((always_inline)) {
        if (mine) {
            const uint32_t tag = static_cast<uint32_t>(nxch + 1);
            float4 part[P];
#pragma unroll
            for (int q = 0; q < P; ++q) {
                if (q == pidx) {
                    part[q] = acc;
                    continue;
                }
                uint64_t* src = xpart(q);
                uint64_t v0 = 0, v1 = 0, v2 = 0, v3 = 0;
                for (int spins = 0; spins < XSPIN && !xbroken; ++spins) {
                    v0 = __hip_atomic_load(src + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    v1 = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    v2 = __hip_atomic_load(src + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    v3 = __hip_atomic_load(src + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (static_cast<uint32_t>(v0 >> 32) == tag && static_cast<uint32_t>(v1 >> 32) == tag &&
                        static_cast<uint32_t>(v2 >> 32) == tag && static_cast<uint32_t>(v3 >> 32) == tag)
                        break;
                    if (spins + 1 == XSPIN) xbroken = true;
                }
                part[q] = make_float4(__uint_as_float(static_cast<uint32_t>(v0)), __uint_as_float(static_cast<uint32_t>(v1)),
                                      __uint_as_float(static_cast<uint32_t>(v2)), __uint_as_float(static_cast<uint32_t>(v3)));
            }
            acc = part[0];
#pragma unroll
            for (int q = 1; q < P; ++q) acc = acc + part[q];
        }
        ++nxch;
        return acc;
    };

    // With split rows and C RPT <= 4, each chunk publishes its part, then prepares
    // the chunk before (which needs no gradient) while the other parts are on
    // their way, and only then waits for them (two prepared chunks live: with
    // C RPT = 8 that spilled).
    constexpr bool PIPE = P > 1 && C * RPT <= 4;
    if constexpr (!PIPE) {
        // Per chunk: prepare, reverse, barrier, sums over waves (over every
        // workgroup's rows where split) and the staged inputs of the chunk before,
        // barrier, the rest.
        for (int n = NC - 1; n >= 0; --n) {
            Prep x;
            prep(x, n, scur);
            float dcv[C][RPT], dkin[C][RPT];
            float4 dZl[RPT];
            reverse(x, n, dcv, dkin, dZl);
            __syncthreads();  // the chunk's partial sums visible
            float4 acc = wave_sums();
            if constexpr (P > 1) {
                publish(acc);
                acc = await_part(acc);
            }
            if (mine) *reinterpret_cast<float4*>(tot + xu * W + xc4 * 4) = acc;
            // the chunk before: its staged inputs and start state (loaded during this chunk)
            if (n > 0) commit(pre, stage_of(n - 1));
#pragma unroll
            for (int i = 0; i < RPT; ++i) scur[i] = pre.st[i];
            __syncthreads();  // the sums over slots and the staged inputs visible
            // (the last chunk loads chunk 0 again: unconditional, no load under a branch)
            issue(pre, n > 1 ? n - 2 : 0);
            finish(x, n, dcv, dkin, dZl);
        }
    } else {
        Prep x;
        prep(x, NC - 1, scur);
        for (int n = NC - 1; n >= 0; --n) {
            float dcv[C][RPT], dkin[C][RPT];
            float4 dZl[RPT];
            reverse(x, n, dcv, dkin, dZl);
            __syncthreads();  // the chunk's partial sums visible
            float4 acc = wave_sums();
            publish(acc);
            if (n > 0) commit(pre, stage_of(n - 1));
#pragma unroll
            for (int i = 0; i < RPT; ++i) scur[i] = pre.st[i];
            __syncthreads();  // the staged inputs of the chunk before visible
            issue(pre, n > 1 ? n - 2 : 0);
            Prep xn;
            if (n > 0) prep(xn, n - 1, scur);
            acc = await_part(acc);
            if (mine) *reinterpret_cast<float4*>(tot + xu * W + xc4 * 4) = acc;
            __syncthreads();  // the sums over slots visible
            finish(x, n, dcv, dkin, dZl);
            if (n > 0) x = xn;
        }
    }

    float* dsi = p.dstate_in + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < RPT; ++i) *reinterpret_cast<float4*>(dsi + el(i)) = dR[i];
}

template <int M, int D, int C, typename TIn, bool DYB, int P>
static void launch_bwd_small_dec(const BwdParams& p, hipStream_t st) {
    // (C = 16: h from the state-passing kernel's fragments)
    constexpr bool CH = C > 8;
    constexpr int NT = bwd_small_threads<M, D, P>();
    const dim3 grid(static_cast<unsigned>(p.f.B) * static_cast<unsigned>(p.f.H) * P);
    if constexpr (P > 1) {
        // the tagged hand-off pairs to zero (tags count the chunks of this call from 1)
        const int nints = static_cast<int>(bwd_small_xchg_bytes(p.f.B, p.f.H, D, P, C) / sizeof(int));
        hipLaunchKernelGGL(osr_bwd_fill_ints<0>, dim3((nints + 255) / 256), dim3(256), 0, st,
                           reinterpret_cast<int*>(p.xbuf), nints);
    }
    // (the first linearisation is its own instantiation, at C <= 8 only)
    if constexpr (C <= 8) {
        if (p.f.lin1) {
            if (p.f.mode == 0)
                hipLaunchKernelGGL((osr_bwd_small_kernel<M, D, NT, C, TIn, DYB, true, P, CH, true>), grid, dim3(NT), 0,
                                   st, p);
            else
                hipLaunchKernelGGL((osr_bwd_small_kernel<M, D, NT, C, TIn, DYB, false, P, false, true>), grid, dim3(NT),
                                   0, st, p);
            return;
        }
    }
    if (p.f.mode == 0)
        hipLaunchKernelGGL((osr_bwd_small_kernel<M, D, NT, C, TIn, DYB, true, P, CH>), grid, dim3(NT), 0, st, p);
    else
        hipLaunchKernelGGL((osr_bwd_small_kernel<M, D, NT, C, TIn, DYB, false, P>), grid, dim3(NT), 0, st, p);
}

// (C = 16 follows the state-passing kernel, which takes bf16 inputs only)
template <int M, int D, int C, int P>
static void launch_bwd_small_p(const BwdParams& p, bool in_bf16, hipStream_t st) {
    if (in_bf16) {
        if (p.dy_bf16)
            launch_bwd_small_dec<M, D, C, uint16_t, true, P>(p, st);
        else
            launch_bwd_small_dec<M, D, C, uint16_t, false, P>(p, st);
    } else if constexpr (C <= 8) {
        if (p.dy_bf16)
            launch_bwd_small_dec<M, D, C, float, true, P>(p, st);
        else
            launch_bwd_small_dec<M, D, C, float, false, P>(p, st);
    }
}

// P (p.split_p) = 2 or 4: the rows of a sequence over P workgroups, with the
// hand-off buffers at p.xbuf (bwd_small_xchg_bytes; the host ensures B*H*P
// workgroups are resident at once).
template <int M, int D, int C>
static int launch_bwd_small_mdc(const BwdParams& p, bool in_bf16, hipStream_t st) {
    if constexpr (!bwd_small_fits<M, D>(C)) {
        return -3;
    } else {
        if (p.split_p == 2) {
            if constexpr (bwd_small_split_ok<M, D, C, 2>()) {
                if (p.xbuf == nullptr) return -3;
                launch_bwd_small_p<M, D, C, 2>(p, in_bf16, st);
            } else {
                return -3;
            }
        } else if (p.split_p == 4) {
            if constexpr (bwd_small_split_ok<M, D, C, 4>()) {
                if (p.xbuf == nullptr) return -3;
                launch_bwd_small_p<M, D, C, 4>(p, in_bf16, st);
            } else {
                return -3;
            }
        } else if (p.split_p == 1) {
            if constexpr (bwd_small_split_ok<M, D, C, 1>())
                launch_bwd_small_p<M, D, C, 1>(p, in_bf16, st);
            else
                return -3;
        } else {
            return -3;
        }
        return hipGetLastError() == hipSuccess ? 0 : -5;
    }
}

template <int M, int D>
int launch_bwd_small_md(const BwdParams& p, bool in_bf16, hipStream_t st) {
    switch (p.f.chunk) {
        case 1: return launch_bwd_small_mdc<M, D, 1>(p, in_bf16, st);
        case 2: return launch_bwd_small_mdc<M, D, 2>(p, in_bf16, st);
        case 4: return launch_bwd_small_mdc<M, D, 4>(p, in_bf16, st);
        case 8: return launch_bwd_small_mdc<M, D, 8>(p, in_bf16, st);
        case 16: return launch_bwd_small_mdc<M, D, 16>(p, in_bf16, st);
        default: return -3;
    }
}

template <int M, int D>
bool bwd_small_split_ok_md(int C, int P) {
    auto ok = [&](auto c) {
        constexpr int CV = decltype(c)::value;
        return (P == 1 && bwd_small_split_ok<M, D, CV, 1>()) || (P == 2 && bwd_small_split_ok<M, D, CV, 2>()) ||
               (P == 4 && bwd_small_split_ok<M, D, CV, 4>());
    };
    switch (C) {
        case 1: return ok(std::integral_constant<int, 1>{});
        case 2: return ok(std::integral_constant<int, 2>{});
        case 4: return ok(std::integral_constant<int, 4>{});
        case 8: return ok(std::integral_constant<int, 8>{});
        case 16: return ok(std::integral_constant<int, 16>{});
        default: return false;
    }
}

template <int M>
bool bwd_small_split_ok_m(int d, int C, int P) {
    switch (d) {
        case 16: return bwd_small_split_ok_md<M, 16>(C, P);
        case 32: return bwd_small_split_ok_md<M, 32>(C, P);
        case 64: return bwd_small_split_ok_md<M, 64>(C, P);
        case 128: return bwd_small_split_ok_md<M, 128>(C, P);
        default: return false;
    }
}

template <int M>
bool bwd_small_fits_m(int d, int C) {
    switch (d) {
        case 16: return bwd_small_fits<M, 16>(C);
        case 32: return bwd_small_fits<M, 32>(C);
        case 64: return bwd_small_fits<M, 64>(C);
        case 128: return bwd_small_fits<M, 128>(C);
        default: return false;
    }
}

}  // namespace osr
