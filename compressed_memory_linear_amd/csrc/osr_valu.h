// osr_valu.h -- register layout and reductions of the VALU (fp32) OSR
// kernels: the decode step and token loop (osr_valu.hip) and the backward
// (osr_bwd.hip).
//
// Thread layout: the m x d fp32 state lives in registers.  TPR = d/4 threads
// cover one slot row with float4 columns; NT/TPR row groups take rows
// rg, rg + RG, ...  Reductions over d stay inside a group of TPR consecutive
// lanes (shuffles); reductions over slots go across row groups (shuffles,
// then one LDS exchange across waves).
#pragma once

#include "osr_device.h"

namespace osr {

template <int M, int D, int NT>
struct ValuLayout {
    static constexpr int TPR = D / 4;         // threads per slot row
    static constexpr int RG = NT / TPR;       // row groups
    static constexpr int RPT = M / RG;        // rows per thread
    static constexpr int NW = NT / 64;        // waves
    static_assert(NT % 64 == 0, "whole waves");
    static_assert(TPR >= 1 && TPR <= 32 && 64 % TPR == 0, "row group inside a wave");
    static_assert(RG * RPT == M && RPT >= 1, "rows divide evenly");
};

template <int RPT>
struct TokenIn {
    float k[RPT], q[RPT], g[RPT];
    float4 v;
    float mu;
};

// Column sums (over slots) of a per-thread float4 partial.  Uses red[NW*D]
// and one barrier (see osr_token for how callers rotate buffers).
template <class L, int D>
__device__ __forceinline__ float4 col_sum(float4 p, float* red, int lane, int wave, int cg) {
    if constexpr (L::TPR < 64) {
        p.x = strided_sum<L::TPR>(p.x);
        p.y = strided_sum<L::TPR>(p.y);
        p.z = strided_sum<L::TPR>(p.z);
        p.w = strided_sum<L::TPR>(p.w);
    }
    if constexpr (L::NW == 1) {
        return p;
    } else {
        if (lane < L::TPR) *reinterpret_cast<float4*>(red + wave * D + cg * 4) = p;
        __syncthreads();
        float4 s = *reinterpret_cast<const float4*>(red + cg * 4);
#pragma unroll
        for (int w = 1; w < L::NW; ++w) s = s + *reinterpret_cast<const float4*>(red + w * D + cg * 4);
        return s;
    }
}

template <class L, int M, int D, typename TIn>
__device__ __forceinline__ void load_token(TokenIn<L::RPT>& in, const Params& p, int64_t bth,
                                           int rg, int cg) {
    const TIn* q = static_cast<const TIn*>(p.q);
    const TIn* k = static_cast<const TIn*>(p.k);
    const TIn* g = static_cast<const TIn*>(p.gamma);
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        const int row = rg + L::RG * i;
        in.k[i] = ld<TIn>(k, bth * M + row);
        in.q[i] = ld<TIn>(q, bth * M + row);
        // one load at a selected index: a load on either arm of a branch would be
        // waited for where the arms join, which undoes any prefetch of the token
        in.g[i] = ld<TIn>(g, p.gamma_per_slot ? bth * M + row : bth);
    }
    in.v = ld4<TIn>(static_cast<const TIn*>(p.v), bth * D + cg * 4);
    in.mu = ld<TIn>(static_cast<const TIn*>(p.mu), bth);
}

// Row sums of squares -> scale every row onto the unit sphere.
template <class L>
__device__ __forceinline__ void project_rows(float4 (&s)[L::RPT]) {
    float n2[L::RPT];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) n2[i] = dot4(s[i], s[i]);
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) n2[i] = group_sum<L::TPR>(n2[i]);
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) s[i] = rsqrtf(n2[i]) * s[i];
}


// Threads per workgroup of the token loops at (M, D): one float4 of a state
// row per thread, at most 512 threads.
template <int M, int D>
constexpr int tokenloop_threads() {
    return (M * (D / 4) < 512) ? M * (D / 4) : 512;
}

// Tokens per batched exchange over slots (the backward's reverse walk keeps 3
// values per slot row and token of a batch in registers).
template <class L>
struct TokBatch {
    static constexpr int BT_REG = L::RPT <= 2 ? 8 : (L::RPT <= 4 ? 4 : 2);
    // at d = 128 at most 4, so that the exchange buffers and a chunk's h fit in LDS
    static constexpr int BT = (L::TPR == 32 && BT_REG > 4) ? 4 : BT_REG;
};

// h of every token of the chunk [t0, t0 + C) into hbuf[C][D] (fp32), from the
// projected chunk-start state z.  Decoding objective: h = sum_i k_i z_i - v,
// the sum over slots exchanged through red once per BT tokens; otherwise -v
// or v.  Ends with a barrier (hbuf visible to all threads).
template <class L, int M, int D, typename TIn>
__device__ __forceinline__ void chunk_h(const float4 (&z)[L::RPT], const Params& f, int64_t bth0,
                                        int64_t tstride, int C, int mode, float* hbuf, float* red,
                                        int& nred, int tid, int lane, int wave, int rg, int cg) {
    constexpr int BT = TokBatch<L>::BT, W = D + 4, Q = D / 4;
    static_assert(BT * Q <= L::NW * 64, "one output float4 per thread");
    const TIn* kp = static_cast<const TIn*>(f.k);
    const TIn* vp = static_cast<const TIn*>(f.v);
    if (mode != 0) {
        const float sgn = mode == 2 ? 1.f : -1.f;
        for (int idx = tid; idx < C * Q; idx += L::NW * 64) {
            const int u = idx / Q, c4 = idx % Q;
            *reinterpret_cast<float4*>(hbuf + u * D + c4 * 4) = sgn * ld4<TIn>(vp, (bth0 + u * tstride) * D + c4 * 4);
        }
        __syncthreads();
        return;
    }
    const int nb = C < BT ? C : BT;
    for (int u0 = 0; u0 < C; u0 += nb) {
        float* rb = red + (nred++ & 1) * (BT * L::NW * W);
        // Every load of the batch is issued before any is used, and none under a
        // branch (indices past the batch repeat its last token): a load inside a
        // branch is waited for where the branch joins, one latency per token.
        float kv[BT][L::RPT];
#pragma unroll
        for (int u = 0; u < BT; ++u) {
            const int64_t bth = bth0 + (u0 + (u < nb ? u : nb - 1)) * tstride;
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) kv[u][i] = ld<TIn>(kp, bth * M + rg + L::RG * i);
        }
        const int uo = tid / Q < nb ? tid / Q : nb - 1, co = tid % Q;  // this thread's output float4
        const float4 vo = ld4<TIn>(vp, (bth0 + (u0 + uo) * tstride) * D + co * 4);
#pragma unroll
        for (int u = 0; u < BT; ++u) {
            if (u < nb) {
                float4 hp = f4(0.f);
#pragma unroll
                for (int i = 0; i < L::RPT; ++i) hp = fma4(kv[u][i], z[i], hp);
                hp.x = strided_sum<L::TPR>(hp.x);
                hp.y = strided_sum<L::TPR>(hp.y);
                hp.z = strided_sum<L::TPR>(hp.z);
                hp.w = strided_sum<L::TPR>(hp.w);
                if (lane < L::TPR) *reinterpret_cast<float4*>(rb + (u * L::NW + wave) * W + cg * 4) = hp;
            }
        }
        __syncthreads();
        if (tid < nb * Q) {
            float4 acc = *reinterpret_cast<const float4*>(rb + (uo * L::NW) * W + co * 4);
#pragma unroll
            for (int w = 1; w < L::NW; ++w) acc = acc + *reinterpret_cast<const float4*>(rb + (uo * L::NW + w) * W + co * 4);
            *reinterpret_cast<float4*>(hbuf + (u0 + uo) * D + co * 4) = acc - vo;
        }
    }
    __syncthreads();
}

}  // namespace osr
