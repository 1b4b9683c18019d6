// osr_bwd.hip -- backward of the chunk-wise OSR forward on gfx950 (fp32 VALU).
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646).  The layer is trained through its chunk-wise form (section
// "Parallel and Hardware Efficient Form", eq. recurrence_linear2); this kernel
// returns the vector-Jacobian product of that forward at chunk size C (exact
// recurrence at C = 1): given dy and the gradient of the returned state, the
// gradients of q, k, v, gamma, mu and the initial state.
//
// Forward per token t of a chunk (Z = unit-projected chunk-start state, R the
// running state, rows = slots):
//   h = sum_i k_i z_i - v | -v | v      c_i = z_i . h      hh = |h|^2
//   a_i = gamma_i k_i (encoding layer: gamma_i (c_i - k_i))
//   w_i = max(hh - c_i^2, 0)            beta_i = (mu^2 + a_i^2 w_i)^(-1/2)
//   g_i = beta_i (mu + a_i c_i)         kap_i = -beta_i a_i
//   r_i <- g_i r_i + kap_i h            y = sum_i q_i r_i
// Reverse of one token, with dR the gradient of the state after the token:
//   dq_i = r_i . dy;  dR_i += q_i dy
//   dg_i = r_prev_i . dR_i;  dkap_i = h . dR_i
//   (beta, a, c, mu) from (dg, dkap) by the chain rule through g and kap,
//   then through beta = (mu^2 + a^2 w)^(-1/2) and w (only where w > 0)
//   dh = sum_i (kap_i dR_i + dc_i z_i) + 2 h dhh
//   dZ_i += dc_i h (+ k_i dh, decoding objective: dk_i += z_i . dh)
//   dv = -dh (decoding, similarity) or dh (encoding layer)
//   dR_i <- g_i dR_i
// At the chunk start dZ + dR (the gradient of Z) goes back through the
// projection onto the sphere: dS_i = (dz_i - z_i (z_i . dz_i)) / |s_i|.
//
// One workgroup per (b,h), state in registers in the layout of osr_valu.h.
// Phase 1 runs the forward and keeps every chunk-start state (before
// projection) in the workspace.  Phase 2 walks the chunks backwards: it runs
// the chunk forward again from its stored start, keeping the state before
// each token and the per-token c, beta, h, |h|^2 in the workspace, then walks
// the chunk's tokens backwards.
#include "osr_launch.h"
#include "osr_valu.h"

namespace osr {

// Per-token record kept for the reverse walk: c[M], beta[M], h[D], |h|^2, pad.
template <int M, int D>
struct TokRec {
    static constexpr int C_OFF = 0, B_OFF = M, H_OFF = 2 * M, HH_OFF = 2 * M + D;
    static constexpr int SIZE = 2 * M + D + 4;
};

template <int M, int D>
__host__ __device__ inline int64_t bwd_floats_per_bh(int T, int C) {
    return (static_cast<int64_t>(T / C) + 1 + C) * M * D + static_cast<int64_t>(C) * TokRec<M, D>::SIZE;
}

// One forward token at the chunk-start state z: updates r and returns the
// per-slot c and beta and h, |h|^2 (all valid in every thread of a row group).
template <class L, int D>
__device__ __forceinline__ void fwd_token_keep(const float4 (&z)[L::RPT], float4 (&r)[L::RPT],
                                               const TokenIn<L::RPT>& in, int mode, float* red,
                                               int lane, int wave, int cg, float (&c)[L::RPT],
                                               float (&beta)[L::RPT], float4& h, float& hh) {
    if (mode == 0) {
        float4 hp = f4(0.f);
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) hp = fma4(in.k[i], z[i], hp);
        h = col_sum<L, D>(hp, red, lane, wave, cg) - in.v;
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
    hh = cc[L::RPT];
    const float mu = in.mu;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        const float a = in.g[i] * (mode == 2 ? cc[i] - in.k[i] : in.k[i]);
        const float w = fmaxf(fmaf(-cc[i], cc[i], hh), 0.f);
        const float b = rsqrtf(fmaf(mu, mu, a * a * w));
        r[i] = fma4(b * fmaf(a, cc[i], mu), r[i], (-b * a) * h);
        c[i] = cc[i];
        beta[i] = b;
    }
}

// Sum over all slots of a per-thread float4 column partial and of a float4 of
// per-slot scalars (every lane of a row group holds the same scalars, so one
// lane per row group is counted).  The result is valid in every thread.  Uses
// red[NW*(D+4)] and one barrier; consecutive calls alternate buffers.
template <class L, int D>
__device__ __forceinline__ void slot_sum2(float4& col, float4& sc, float* red, int lane, int wave, int cg) {
    if constexpr (L::TPR < 64) {
        col.x = strided_sum<L::TPR>(col.x);
        col.y = strided_sum<L::TPR>(col.y);
        col.z = strided_sum<L::TPR>(col.z);
        col.w = strided_sum<L::TPR>(col.w);
        sc.x = strided_sum<L::TPR>(sc.x);
        sc.y = strided_sum<L::TPR>(sc.y);
        sc.z = strided_sum<L::TPR>(sc.z);
    }
    if constexpr (L::NW > 1) {
        constexpr int W = D + 4;
        if (lane < L::TPR) *reinterpret_cast<float4*>(red + wave * W + cg * 4) = col;
        if (lane == 0) *reinterpret_cast<float4*>(red + wave * W + D) = sc;
        __syncthreads();
        float4 s = *reinterpret_cast<const float4*>(red + cg * 4);
        float4 t = *reinterpret_cast<const float4*>(red + D);
#pragma unroll
        for (int w = 1; w < L::NW; ++w) {
            s = s + *reinterpret_cast<const float4*>(red + w * W + cg * 4);
            t = t + *reinterpret_cast<const float4*>(red + w * W + D);
        }
        col = s;
        sc = t;
    }
}

// What the reverse walk reads for one token: its inputs, its record, dy and
// (when prefetched) the state before it.
template <int RPT>
struct RevIn {
    TokenIn<RPT> in;
    float c[RPT], beta[RPT];
    float4 h, dy;
    float hh;
    float4 rp[RPT];
};

template <class L, int M, int D, typename TIn, bool PF_STATE>
__device__ __forceinline__ void load_rev(RevIn<L::RPT>& x, const BwdParams& p, const float* trec,
                                         const float* rtok, int64_t bth, int tau, int rg, int cg, int el0) {
    using TR = TokRec<M, D>;
    load_token<L, M, D, TIn>(x.in, p.f, bth, rg, cg);
    const float* rec = trec + static_cast<int64_t>(tau) * TR::SIZE;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        x.c[i] = rec[TR::C_OFF + rg + L::RG * i];
        x.beta[i] = rec[TR::B_OFF + rg + L::RG * i];
    }
    x.h = *reinterpret_cast<const float4*>(rec + TR::H_OFF + cg * 4);
    x.hh = rec[TR::HH_OFF];
    x.dy = p.dy_bf16 ? ld4<uint16_t>(static_cast<const uint16_t*>(p.dy), bth * D + cg * 4)
                     : ld4<float>(static_cast<const float*>(p.dy), bth * D + cg * 4);
    if constexpr (PF_STATE) {
        const float* rpre = rtok + static_cast<int64_t>(tau) * M * D;
#pragma unroll
        for (int i = 0; i < L::RPT; ++i)
            x.rp[i] = *reinterpret_cast<const float4*>(rpre + el0 + i * L::RG * D);
    }
}

template <int M, int D, int NT, typename TIn>
__global__ __launch_bounds__(NT) void osr_bwd_kernel(BwdParams p) {
    using L = ValuLayout<M, D, NT>;
    using TR = TokRec<M, D>;
    // The reverse walk loads the next token's inputs and record while it works on
    // the current one, and the state before it too, where registers allow (at
    // 8 slot rows per thread either would spill).
    constexpr bool PF_TOKEN = L::RPT <= 4;
    constexpr bool PF_STATE = L::RPT <= 2;
    __shared__ float red[2][L::NW * (D + 4)];
    const int bh = blockIdx.x;
    const int b = bh / p.f.H, hd = bh % p.f.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % L::TPR, rg = tid / L::TPR;
    const int T = p.f.T, C = p.f.chunk, NC = T / C;
    const int mode = p.f.mode;

    float* ws = p.ws + static_cast<int64_t>(bh) * bwd_floats_per_bh<M, D>(T, C);
    float* sck = ws;                                          // [NC+1][M][D]
    float* rtok = sck + static_cast<int64_t>(NC + 1) * M * D;  // [C][M][D]
    float* trec = rtok + static_cast<int64_t>(C) * M * D;      // [C][TR::SIZE]
    auto el = [&](int i) { return (rg + L::RG * i) * D + cg * 4; };  // this thread's state elements
    auto bth_of = [&](int t) { return (static_cast<int64_t>(b) * T + t) * p.f.H + hd; };
    int nred = 0;  // LDS reductions so far: consecutive ones use alternate buffers

    // ---- phase 1: forward, keeping every chunk-start state ----
    float4 r[L::RPT], z[L::RPT];
    const float* sin = p.f.state_in + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) r[i] = *reinterpret_cast<const float4*>(sin + el(i));
    TokenIn<L::RPT> cur, nxt;
    if constexpr (PF_TOKEN) load_token<L, M, D, TIn>(cur, p.f, bth_of(0), rg, cg);
    for (int n = 0; n < NC; ++n) {
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) *reinterpret_cast<float4*>(sck + static_cast<int64_t>(n) * M * D + el(i)) = r[i];
        project_rows<L>(r);
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) z[i] = r[i];
        for (int t = n * C; t < (n + 1) * C; ++t) {
            if constexpr (PF_TOKEN) {
                if (t + 1 < T) load_token<L, M, D, TIn>(nxt, p.f, bth_of(t + 1), rg, cg);
            } else {
                load_token<L, M, D, TIn>(cur, p.f, bth_of(t), rg, cg);
            }
            float c[L::RPT], beta[L::RPT], hh;
            float4 h;
            fwd_token_keep<L, D>(z, r, cur, mode, red[nred & 1], lane, wave, cg, c, beta, h, hh);
            nred += mode == 0;  // only the decoding objective reduces over slots here
            if constexpr (PF_TOKEN) cur = nxt;
        }
    }
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) *reinterpret_cast<float4*>(sck + static_cast<int64_t>(NC) * M * D + el(i)) = r[i];

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
        __syncthreads();  // the previous chunk's reverse walk has read rtok / trec
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
        // forward again over the chunk, keeping what the reverse walk needs
        if constexpr (PF_TOKEN) load_token<L, M, D, TIn>(cur, p.f, bth_of(n * C), rg, cg);
        for (int tau = 0; tau < C; ++tau) {
#pragma unroll
            for (int i = 0; i < L::RPT; ++i)
                *reinterpret_cast<float4*>(rtok + static_cast<int64_t>(tau) * M * D + el(i)) = r[i];
            if constexpr (PF_TOKEN) {
                if (tau + 1 < C) load_token<L, M, D, TIn>(nxt, p.f, bth_of(n * C + tau + 1), rg, cg);
            } else {
                load_token<L, M, D, TIn>(cur, p.f, bth_of(n * C + tau), rg, cg);
            }
            float c[L::RPT], beta[L::RPT], hh;
            float4 h;
            fwd_token_keep<L, D>(z, r, cur, mode, red[nred & 1], lane, wave, cg, c, beta, h, hh);
            if constexpr (PF_TOKEN) cur = nxt;
            nred += mode == 0;  // only the decoding objective reduces over slots here
            float* rec = trec + static_cast<int64_t>(tau) * TR::SIZE;
            if (cg == 0) {
#pragma unroll
                for (int i = 0; i < L::RPT; ++i) {
                    rec[TR::C_OFF + rg + L::RG * i] = c[i];
                    rec[TR::B_OFF + rg + L::RG * i] = beta[i];
                }
            }
            if (rg == 0) *reinterpret_cast<float4*>(rec + TR::H_OFF + cg * 4) = h;
            if (tid == 0) rec[TR::HH_OFF] = hh;
        }
        __syncthreads();  // records visible to every thread

        float4 dZ[L::RPT];
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) dZ[i] = f4(0.f);
        // The state after the chunk's last token is the next chunk's stored start;
        // the state before token tau is the state after token tau - 1.
        float4 rpost[L::RPT];
        if constexpr (PF_STATE) {
            const float* s1 = sck + static_cast<int64_t>(n + 1) * M * D;
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) rpost[i] = *reinterpret_cast<const float4*>(s1 + el(i));
        }
        RevIn<L::RPT> rc, rn;
        if constexpr (PF_TOKEN)
            load_rev<L, M, D, TIn, PF_STATE>(rc, p, trec, rtok, bth_of(n * C + C - 1), C - 1, rg, cg, el(0));
        for (int tau = C - 1; tau >= 0; --tau) {
            const int64_t bth = bth_of(n * C + tau);
            if constexpr (PF_TOKEN) {
                if (tau > 0)
                    load_rev<L, M, D, TIn, PF_STATE>(rn, p, trec, rtok, bth_of(n * C + tau - 1), tau - 1, rg, cg, el(0));
            } else {
                load_rev<L, M, D, TIn, false>(rc, p, trec, rtok, bth, tau, rg, cg, el(0));
            }
            const TokenIn<L::RPT>& in = rc.in;
            const float* c = rc.c;
            const float* beta = rc.beta;
            const float4 h = rc.h;
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

            // reductions over d: dq, dg, dkap
            float dq[L::RPT], dg[L::RPT], dk2[L::RPT];
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) {
                dq[i] = dot4(rpost[i], dy);
                dR[i] = fma4(in.q[i], dy, dR[i]);
                dg[i] = dot4(rp[i], dR[i]);
                dk2[i] = dot4(h, dR[i]);
            }
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) {
                dq[i] = group_sum<L::TPR>(dq[i]);
                dg[i] = group_sum<L::TPR>(dg[i]);
                dk2[i] = group_sum<L::TPR>(dk2[i]);
            }

            // scalar chain rule per slot
            const float mu = in.mu;
            float gate[L::RPT], dc[L::RPT], dkin[L::RPT], dgam[L::RPT];
            float4 hp = f4(0.f);
            float4 sc = f4(0.f);  // (d|h|^2, dmu, dgamma summed over slots, 0)
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) {
                const float coef = mode == 2 ? c[i] - in.k[i] : in.k[i];
                const float a = in.g[i] * coef;
                const float wraw = fmaf(-c[i], c[i], hh);
                const float w = fmaxf(wraw, 0.f);
                const float bt = beta[i];
                const float num = fmaf(a, c[i], mu);
                gate[i] = bt * num;
                const float kap = -bt * a;
                const float dbeta = num * dg[i] - a * dk2[i];
                float da = bt * (c[i] * dg[i] - dk2[i]);
                float dmu_i = bt * dg[i];
                float dci = bt * a * dg[i];
                const float tb = -0.5f * bt * bt * bt * dbeta;
                dmu_i = fmaf(2.f * mu, tb, dmu_i);
                da = fmaf(2.f * a * w, tb, da);
                const float dw = a * a * tb;
                float dhh_i = 0.f;
                if (wraw > 0.f) {
                    dhh_i = dw;
                    dci = fmaf(-2.f * c[i], dw, dci);
                }
                if (mode == 2) {
                    dci = fmaf(in.g[i], da, dci);
                    dkin[i] = -in.g[i] * da;
                    dgam[i] = coef * da;
                } else {
                    dkin[i] = in.g[i] * da;
                    dgam[i] = in.k[i] * da;
                }
                dc[i] = dci;
                hp = fma4(kap, dR[i], fma4(dci, z[i], hp));
                sc.x += dhh_i;
                sc.y += dmu_i;
                sc.z += dgam[i];
            }
            slot_sum2<L, D>(hp, sc, red[nred++ & 1], lane, wave, cg);
            const float4 dh = fma4(2.f * sc.x, h, hp);

            float dkz[L::RPT] = {};
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) {
                dZ[i] = fma4(dc[i], h, dZ[i]);
                if (mode == 0) {
                    dZ[i] = fma4(in.k[i], dh, dZ[i]);
                    dkz[i] = dot4(z[i], dh);
                }
            }
            if (mode == 0) {
#pragma unroll
                for (int i = 0; i < L::RPT; ++i) dkz[i] = group_sum<L::TPR>(dkz[i]);
            }
#pragma unroll
            for (int i = 0; i < L::RPT; ++i) {
                dR[i] = gate[i] * dR[i];
                if constexpr (PF_STATE) rpost[i] = rp[i];
            }

            // stores
            if (cg == 0) {
#pragma unroll
                for (int i = 0; i < L::RPT; ++i) {
                    const int64_t o = bth * M + rg + L::RG * i;
                    p.dq[o] = dq[i];
                    p.dk[o] = mode == 0 ? dkin[i] + dkz[i] : dkin[i];
                    if (p.f.gamma_per_slot) p.dgamma[o] = dgam[i];
                }
            }
            if (tid == 0) {
                p.dmu[bth] = sc.y;
                if (!p.f.gamma_per_slot) p.dgamma[bth] = sc.z;
            }
            if (rg == 0) {
                const float4 dv = mode == 2 ? dh : f4(0.f) - dh;
                *reinterpret_cast<float4*>(p.dv + bth * D + cg * 4) = dv;
            }
            if constexpr (PF_TOKEN) rc = rn;
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

// ----------------------------------------------------------------- launch --
template <int M, int D>
static int launch_bwd_md(const BwdParams& p, bool in_bf16, hipStream_t st) {
    constexpr int TPR = D / 4;
    // 512 threads (1024 at m = d = 128, where 512 would need 8 slot rows per
    // thread and spill).
    constexpr int NT = (M * TPR < 512) ? M * TPR : 512;
    const dim3 grid(static_cast<unsigned>(p.f.B) * static_cast<unsigned>(p.f.H));
    if (in_bf16)
        hipLaunchKernelGGL((osr_bwd_kernel<M, D, NT, uint16_t>), grid, dim3(NT), 0, st, p);
    else
        hipLaunchKernelGGL((osr_bwd_kernel<M, D, NT, float>), grid, dim3(NT), 0, st, p);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int M>
static int launch_bwd_m(int d, const BwdParams& p, bool in_bf16, hipStream_t st) {
    switch (d) {
        case 16: return launch_bwd_md<M, 16>(p, in_bf16, st);
        case 32: return launch_bwd_md<M, 32>(p, in_bf16, st);
        case 64: return launch_bwd_md<M, 64>(p, in_bf16, st);
        case 128: return launch_bwd_md<M, 128>(p, in_bf16, st);
        default: return -3;
    }
}

int launch_bwd(int m, int d, const BwdParams& p, bool in_bf16, hipStream_t st) {
    switch (m) {
        case 16: return launch_bwd_m<16>(d, p, in_bf16, st);
        case 32: return launch_bwd_m<32>(d, p, in_bf16, st);
        case 64: return launch_bwd_m<64>(d, p, in_bf16, st);
        case 128: return launch_bwd_m<128>(d, p, in_bf16, st);
        default: return -3;
    }
}

template <int M>
static size_t bwd_ws_m(int d, int T, int C) {
    switch (d) {
        case 16: return static_cast<size_t>(bwd_floats_per_bh<M, 16>(T, C));
        case 32: return static_cast<size_t>(bwd_floats_per_bh<M, 32>(T, C));
        case 64: return static_cast<size_t>(bwd_floats_per_bh<M, 64>(T, C));
        case 128: return static_cast<size_t>(bwd_floats_per_bh<M, 128>(T, C));
        default: return 0;
    }
}

size_t bwd_workspace_bytes(int B, int H, int T, int m, int d, int C) {
    size_t per = 0;
    switch (m) {
        case 16: per = bwd_ws_m<16>(d, T, C); break;
        case 32: per = bwd_ws_m<32>(d, T, C); break;
        case 64: per = bwd_ws_m<64>(d, T, C); break;
        case 128: per = bwd_ws_m<128>(d, T, C); break;
        default: return 0;
    }
    return per * sizeof(float) * static_cast<size_t>(B) * static_cast<size_t>(H);
}

}  // namespace osr
