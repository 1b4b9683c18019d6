// osr_bwd_chunk.hip -- backward of the chunk-wise OSR forward in its
// chunk-parallel (matrix) form, on the gfx950 fp32 matrix cores.
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646), section "Parallel and Hardware Efficient Form", eq.
// recurrence_linear2.  Inside a chunk every gate, kappa and h_t is taken at
// the unit-projected chunk-start state Z:
//   H = K Z - V (decoding objective; -V for similarity), c = H Z^T,
//   |h_t|^2 = rowsum(H (.) H), a = gamma (.) k, w = max(|h|^2 - c^2, 0),
//   beta = (mu^2 + a^2 w)^(-1/2), kappa = beta a, g = beta (mu + a c),
// and the slots evolve as s_i <- g_i s_i - kappa_i h_t with y_t = sum_i q_i s_i.
// This kernel returns the vector-Jacobian product of that forward with
// respect to q, k, v, gamma, mu and the initial state, given dy and the
// gradient of the returned (projected) end state.
//
// The chunks are taken in reverse, one workgroup per (b,h).  A chunk splits
// into tiles of 16 tokens.  With R_b the state at the start of tile b
// (R_0 = Z) and A the running product of g from the tile start, taken
// relative to a_ref (the product over the tile's first half, which cancels),
//   Y_b = (Q (.) A / a_ref) (a_ref (.) R_b) - tril[(Q A / a_ref)(kappa a_ref / A)^T] H_b
//   R_{b+1} = diag(A_end) R_b - W_b^T H_b,   W_t = kappa_t prod_{l > t in tile} g_l.
// Its backward per chunk, given lambda (the gradient of the chunk-end state):
//   1. recompute Z, H, c, the gates, the tile products and R_1 .. R_{NT-1};
//   2. per tile, independent of lambda: dP = -tril(dY H^T), the gradients of
//      Q A / a_ref and kappa a_ref / A from dP, dH = -P^T dY, and
//      dY (a_ref R_b)^T;
//   3. tiles in reverse: dA_end = rowdot(R_b, lambda), dW = -H_b lambda^T,
//      dH_b -= W_b lambda, lambda <- diag(A_end) lambda + a_ref (.) (Q A / a_ref)^T dY_b;
//   4. per tile: the gradients of A (the reverse recursion E_t = dA_t +
//      g_{t+1} E_{t+1}, dg_t += A_{t-1} E_t: no division by a gate) and of
//      the suffix products of W (a forward recursion), then through beta,
//      kappa and g to c, |h|^2, gamma, k and mu;
//   5. dH += dc Z + 2 diag(d|h|^2) H, dZ = lambda + dc^T H (+ K^T dH),
//      dK += dH Z^T (decoding objective), dV = -dH, and the next lambda is
//      dZ taken back through the chunk-start projection,
//      (dz_i - z_i (z_i . dz_i)) / |s_i|.
// Every product is a v_mfma_f32_16x16x4_f32 chain over LDS operands (fp32
// throughout); the per-(token, slot) values of tile b live in wave b's
// registers in the accumulator layout (lane (lg, lc) holds tokens 4lg..4lg+3
// of slot column lc of each 16-slot block).  The chunk-start states come from
// the state-passing kernel (the backward's workspace holds them).
#include "osr_launch.h"
#include "osr_bwd_kernel.h"

namespace osr {
namespace cbwd {

typedef float f4 __attribute__((ext_vector_type(4)));

constexpr int TL = 16;  // tile length (tokens)

// acc += A[16 x K] B[K x 16] with A(i, k) = a[i * AI + k * AK] and
// B(k, j) = b[k * BK + j * BJ] (LDS, fp32); lane (kq, r) supplies A(r, k0 + kq)
// and B(k0 + kq, r); the result holds rows 4 kq .. 4 kq + 3 of column r.
template <int K, int AI, int AK, int BK, int BJ>
__device__ __forceinline__ f4 mm(f4 acc, const float* a, const float* b, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const float* pa = a + r * AI + kq * AK;
    const float* pb = b + kq * BK + r * BJ;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0 * AK], pb[k0 * BK], acc, 0, 0, 0);
    return acc;
}

// Four output tiles that share the A operand: acc[j] += A B_j with B_j
// starting at b + j * BS (independent accumulation chains, one A load per
// step for four products).
template <int K, int AI, int AK, int BK, int BJ, int BS>
__device__ __forceinline__ void mm4(f4 (&acc)[4], const float* a, const float* b, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const float* pa = a + r * AI + kq * AK;
    const float* pb = b + kq * BK + r * BJ;
#pragma unroll
    for (int k0 = 0; k0 < K; k0 += 4) {
        const float av = pa[k0 * AK];
        float bv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) bv[j] = pb[k0 * BK + j * BS];
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, bv[j], acc[j], 0, 0, 0);
    }
}

__device__ __forceinline__ f4 zero4() { return f4{0.f, 0.f, 0.f, 0.f}; }

// Workgroup barrier for LDS data only: every wave's LDS accesses have
// completed, then s_barrier.  (__syncthreads also waits for the wave's
// global loads and stores; the kernel's global accesses are each thread's own
// -- outputs, and the workspace elements it wrote itself -- so no other wave
// waits for them.)
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Sum over the 16 lanes of a lane row (same lg).
__device__ __forceinline__ float row16_sum(float x) {
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) x += __shfl_xor(x, o, 64);
    return x;
}
// Sum over the 4 consecutive lanes of an element row (the M x D passes).
__device__ __forceinline__ float quad_sum(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    return x;
}

// Affine scans over the 16 tokens of a tile, for one slot column: token
// 4 lg + r of the lane.  Inclusive forward scan of x_t = g_t x_{t-1} + u_t
// (x_{-1} = 0); returns x_t and, in xprev, x_{t-1}.
__device__ __forceinline__ void affine_scan_fwd(const float (&g)[4], const float (&u)[4], float (&x)[4],
                                                float (&xprev)[4], int lane) {
    // the lane's own composition: x_out = G x_in + U
    float G = 1.f, U = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        U = g[r] * U + u[r];
        G *= g[r];
    }
    const int lc = lane & 15, lg = lane >> 4;
    float xin = 0.f;  // x before this lane's first token
#pragma unroll
    for (int j = 0; j < 3; ++j) {
        const float Gj = __shfl(G, lc + 16 * j, 64), Uj = __shfl(U, lc + 16 * j, 64);
        if (j < lg) xin = Gj * xin + Uj;
    }
    float cur = xin;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        xprev[r] = cur;
        cur = g[r] * cur + u[r];
        x[r] = cur;
    }
}
// Reverse: e_t = g_{t+1} e_{t+1} + u_t (e_16 = 0), with gn[r] = g_{t+1}
// (gn of the tile's last token unused).
__device__ __forceinline__ void affine_scan_rev(const float (&gn)[4], const float (&u)[4], float (&e)[4],
                                                int lane) {
    // own composition from the lane's last token down: e_first = G e_after + U
    float G = 1.f, U = 0.f;
#pragma unroll
    for (int r = 3; r >= 0; --r) {
        // e_r = gn[r] e_{r+1} + u[r]: compose e_{r+1} = G' e_after + U'
        U = u[r] + gn[r] * U;
        G = gn[r] * G;
    }
    const int lc = lane & 15, lg = lane >> 4;
    float eafter = 0.f;  // e of the token after this lane's last
#pragma unroll
    for (int j = 3; j >= 1; --j) {
        const float Gj = __shfl(G, lc + 16 * j, 64), Uj = __shfl(U, lc + 16 * j, 64);
        if (j > lg) eafter = Gj * eafter + Uj;
    }
    // the last token of group j has gn = g of the next group's first token,
    // which the composition above already holds for lanes below the top
    float cur = eafter;
#pragma unroll
    for (int r = 3; r >= 0; --r) {
        cur = gn[r] * cur + u[r];
        e[r] = cur;
    }
}

// The gates of one 16-slot block of a tile (lane: tokens 4 lg + r, slot lc)
// and their running products over the tile's 16 tokens: A_t (inclusive),
// A_{t-1}, the suffix products prod_{l > t} g_l, a_ref (the product over the
// first 8 tokens) and A_end.  The same code in both places it runs, so the
// backward's second evaluation repeats the first bit for bit.
struct TileGates {
    float a[4], wv[4], beta[4], kap[4], g[4], A[4], Ap[4], sfx[4];
    float rA[4];    // 1 / A (v_rcp_f32)
    float ar, rar, ae;  // a_ref, 1 / a_ref, A_end
};
__device__ __forceinline__ void tile_gates(const float (&kq)[4], const float (&gm)[4], const float (&mu)[4],
                                           const float (&hh)[4], const float (&ht)[4], int lane, TileGates& o) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const float a = gm[r] * kq[r];
        const float wr = hh[r] - ht[r] * ht[r];
        const float wv = wr > 0.f ? wr : 0.f;
        const float bt = rsqrtf(mu[r] * mu[r] + a * a * wv);
        o.a[r] = a;
        o.wv[r] = wv;
        o.beta[r] = bt;
        o.kap[r] = bt * a;
        o.g[r] = bt * (mu[r] + a * ht[r]);
    }
    const int lc = lane & 15, lg = lane >> 4;
    float lp = 1.f, lprod[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        lp *= o.g[r];
        lprod[r] = lp;
    }
    float tot[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) tot[j] = __shfl(lp, lc + 16 * j, 64);
    float below = 1.f, above = 1.f;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        if (j < lg) below *= tot[j];
        if (j > lg) above *= tot[j];
    }
    o.ar = tot[0] * tot[1];
    o.ae = tot[0] * tot[1] * tot[2] * tot[3];
    float ls = 1.f;
#pragma unroll
    for (int r = 3; r >= 0; --r) {
        o.sfx[r] = ls * above;
        ls *= o.g[r];
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        o.A[r] = below * lprod[r];
        o.Ap[r] = r == 0 ? below : below * lprod[r - 1];
        o.rA[r] = __builtin_amdgcn_rcpf(o.A[r]);
    }
    o.rar = __builtin_amdgcn_rcpf(o.ar);
}

template <int M, int D, int C, typename TIn, bool DYB>
struct Cfg {
    static constexpr int LDX = 68;  // row stride (floats) of the LDS matrices
    static constexpr int NT = C / TL;
    static constexpr int NW = NT;   // wave b holds tile b
    static constexpr int MT = M / 16, DT = D / 16;
    static_assert(M == 64 && D == 64 && C == 64, "built for m = d = C = 64");
    static_assert(MT == NW, "the M x D products give wave w the slot block w");
};

template <int M, int D, int C, typename TIn, bool DYB>
__global__ __launch_bounds__(256) void osr_bwd_chunk_kernel(BwdParams p) {
    using G = Cfg<M, D, C, TIn, DYB>;
    constexpr int LDX = G::LDX, NT = G::NT, MT = G::MT, DT = G::DT;
    __shared__ __attribute__((aligned(16))) float Zs[M * LDX];   // Z
    __shared__ __attribute__((aligned(16))) float Hs[C * LDX];   // H
    __shared__ __attribute__((aligned(16))) float Ys[C * LDX];   // dY
    __shared__ __attribute__((aligned(16))) float Us[C * LDX];   // V, then dH
    __shared__ __attribute__((aligned(16))) float Ls[M * LDX];   // R_b, then lambda, then dZ
    __shared__ __attribute__((aligned(16))) float QAs[C * LDX];  // Q A / a_ref, then dc
    __shared__ __attribute__((aligned(16))) float KAs[C * LDX];  // kappa a_ref / A, then K
    __shared__ __attribute__((aligned(16))) float Ws[C * LDX];   // K, then W
    __shared__ float Ps[NT][16 * 17], dPs[NT][16 * 17];          // per tile: P, dP ([t][u])
    __shared__ float nh_s[C], dnh_s[C], ae_s[NT * M], ar_s[NT * M], dae_s[NT * M], invn_s[M];

    const int bh = blockIdx.x, b = bh / p.f.H, hd = bh % p.f.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lg = lane >> 4, lc = lane & 15;
    const int T = p.f.T, NC = T / C;
    const bool dec = p.f.mode == 0;
    const bool gps = p.f.gamma_per_slot != 0;
    const TIn* qp = static_cast<const TIn*>(p.f.q);
    const TIn* kp = static_cast<const TIn*>(p.f.k);
    const TIn* vp = static_cast<const TIn*>(p.f.v);
    const TIn* gp = static_cast<const TIn*>(p.f.gamma);
    const TIn* mp = static_cast<const TIn*>(p.f.mu);
    float* ws = p.ws + static_cast<int64_t>(bh) * bwd_floats_per_bh<M, D>(T, C);
    const float* sck = ws;                                      // [NC+1][M][D] chunk-start states
    float* rst = ws + static_cast<int64_t>(NC + 1) * M * D;     // [NT][M][D] tile-start states
    auto bth = [&](int t) { return (static_cast<int64_t>(b) * T + t) * p.f.H + hd; };

    // M x D element passes: row er, columns 16 ec .. 16 ec + 15
    const int er = tid >> 2, ec = tid & 3;
    float lam[16];  // lambda (gradient of the chunk-end state) between chunks, this thread's elements

    // the returned state is the end state projected: its backward
    {
        const float* s = sck + static_cast<int64_t>(NC) * M * D + er * D + 16 * ec;
        const float* g = p.dstate_out + static_cast<int64_t>(bh) * M * D + er * D + 16 * ec;
        float sv[16], n2 = 0.f, pr = 0.f;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            sv[j] = s[j];
            lam[j] = g[j];
            n2 += sv[j] * sv[j];
        }
        const float inv = rsqrtf(quad_sum(n2));
#pragma unroll
        for (int j = 0; j < 16; ++j) pr += sv[j] * inv * lam[j];
        pr = quad_sum(pr);
#pragma unroll
        for (int j = 0; j < 16; ++j) lam[j] = inv * (lam[j] - pr * sv[j] * inv);
    }

    {
        // lambda lives in the workspace between chunks (each thread its own elements)
        float* dst = rst + static_cast<int64_t>(NT) * M * D + er * D + 16 * ec;
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[j] = lam[j];
    }
    const int t_lane = 4 * lg;  // first token (within the tile) of this lane's rows
    for (int n = NC - 1; n >= 0; --n) {
        const int tc = n * C + TL * w;  // first token of this wave's tile
        // ---- 1. Z, V, dY, K into LDS; this tile's inputs into registers ----
        {
            const float* s = sck + static_cast<int64_t>(n) * M * D + er * D + 16 * ec;
            float sv[16], n2 = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                sv[j] = s[j];
                n2 += sv[j] * sv[j];
            }
            const float inv = rsqrtf(quad_sum(n2));
#pragma unroll
            for (int j = 0; j < 16; ++j) Zs[er * LDX + 16 * ec + j] = sv[j] * inv;
            if (ec == 0) invn_s[er] = inv;
            // token rows: V and dY [C][D], K [C][M] (er is the token here)
            const int64_t tv = bth(n * C + er);
#pragma unroll
            for (int j = 0; j < 16; j += 4) {
                const float4 v4 = ld4<TIn>(vp, tv * D + 16 * ec + j);
                Us[er * LDX + 16 * ec + j + 0] = v4.x;
                Us[er * LDX + 16 * ec + j + 1] = v4.y;
                Us[er * LDX + 16 * ec + j + 2] = v4.z;
                Us[er * LDX + 16 * ec + j + 3] = v4.w;
                float4 y4;
                if constexpr (DYB)
                    y4 = ld4<uint16_t>(static_cast<const uint16_t*>(p.dy), tv * D + 16 * ec + j);
                else
                    y4 = ld4<float>(static_cast<const float*>(p.dy), tv * D + 16 * ec + j);
                Ys[er * LDX + 16 * ec + j + 0] = y4.x;
                Ys[er * LDX + 16 * ec + j + 1] = y4.y;
                Ys[er * LDX + 16 * ec + j + 2] = y4.z;
                Ys[er * LDX + 16 * ec + j + 3] = y4.w;
                const float4 k4 = ld4<TIn>(kp, tv * M + 16 * ec + j);
                Ws[er * LDX + 16 * ec + j + 0] = k4.x;
                Ws[er * LDX + 16 * ec + j + 1] = k4.y;
                Ws[er * LDX + 16 * ec + j + 2] = k4.z;
                Ws[er * LDX + 16 * ec + j + 3] = k4.w;
            }
        }
        // this tile's mu (token tc + t_lane + r); its q, k, gamma are loaded per
        // slot block where they are used (slot 16 mt + lc)
        float mu[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) mu[r] = ld<TIn>(mp, bth(tc + t_lane + r));
        auto load_in = [&](int mt, float (&kq)[4], float (&qv)[4], float (&gm)[4]) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t tt = bth(tc + t_lane + r);
                kq[r] = ld<TIn>(kp, tt * M + 16 * mt + lc);
                qv[r] = ld<TIn>(qp, tt * M + 16 * mt + lc);
                gm[r] = gps ? ld<TIn>(gp, tt * M + 16 * mt + lc) : ld<TIn>(gp, tt);
            }
        };
        lds_barrier();

        // ---- 2. H = K Z - V for this wave's tile; |h|^2 ----
        float hh[4] = {0.f, 0.f, 0.f, 0.f};
        {
            f4 acc[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[dt][r] = -Us[(TL * w + t_lane + r) * LDX + 16 * dt + lc];
            if (dec) mm4<M, LDX, 1, LDX, 1, 16>(acc, Ws + TL * w * LDX, Zs, lane);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Hs[(TL * w + t_lane + r) * LDX + 16 * dt + lc] = acc[dt][r];
                    hh[r] += acc[dt][r] * acc[dt][r];
                }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) hh[r] = row16_sum(hh[r]);
        if (lc == 0)
#pragma unroll
            for (int r = 0; r < 4; ++r) nh_s[TL * w + t_lane + r] = hh[r];
        lds_barrier();  // H visible; every wave is done with K in Ws

        // ---- 3. c = H Z^T (this tile) and the gates ----
        float ht[MT][4];
        float kq3[MT][4], qv3[MT][4], gm3[MT][4];  // this tile's inputs, loaded before the product
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) load_in(mt, kq3[mt], qv3[mt], gm3[mt]);
        {
            f4 acc[MT] = {zero4(), zero4(), zero4(), zero4()};
            mm4<D, LDX, 1, 1, LDX, 16 * LDX>(acc, Hs + TL * w * LDX, Zs, lane);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) ht[mt][r] = acc[mt][r];
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            TileGates tg;
            tile_gates(kq3[mt], gm3[mt], mu, hh, ht[mt], lane, tg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (TL * w + t_lane + r) * LDX + 16 * mt + lc;
                QAs[o] = qv3[mt][r] * tg.A[r] * tg.rar;
                KAs[o] = tg.kap[r] * tg.ar * tg.rA[r];
                Ws[o] = tg.kap[r] * tg.sfx[r];
            }
            if (lg == 0) {
                ae_s[w * M + 16 * mt + lc] = tg.ae;
                ar_s[w * M + 16 * mt + lc] = tg.ar;
            }
        }
        lds_barrier();

        // ---- 4. per tile: P, dP and the lambda-free gradients ----
        {
            const f4 pa = mm<M, LDX, 1, 1, LDX>(zero4(), QAs + TL * w * LDX, KAs + TL * w * LDX, lane);
            const f4 pd = mm<D, LDX, 1, 1, LDX>(zero4(), Ys + TL * w * LDX, Hs + TL * w * LDX, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool causal = lc <= t_lane + r;  // u <= t
                Ps[w][(t_lane + r) * 17 + lc] = causal ? pa[r] : 0.f;
                dPs[w][(t_lane + r) * 17 + lc] = causal ? -pd[r] : 0.f;
            }
        }
        lds_barrier();
        float dqa[MT][4], dka[MT][4];
        {
            // dQA' = dP KA', dKA' = dP^T QA', dH = -P^T dY (into Us: V is dead since step 2)
            f4 x[MT] = {zero4(), zero4(), zero4(), zero4()}, y[MT] = {zero4(), zero4(), zero4(), zero4()};
            f4 z[DT] = {zero4(), zero4(), zero4(), zero4()};
            mm4<TL, 17, 1, LDX, 1, 16>(x, dPs[w], KAs + TL * w * LDX, lane);
            mm4<TL, 1, 17, LDX, 1, 16>(y, dPs[w], QAs + TL * w * LDX, lane);
            mm4<TL, 1, 17, LDX, 1, 16>(z, Ps[w], Ys + TL * w * LDX, lane);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dqa[mt][r] = x[mt][r];
                    dka[mt][r] = y[mt][r];
                }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) Us[(TL * w + t_lane + r) * LDX + 16 * dt + lc] = -z[dt][r];
        }

        // ---- 5. tile-start states R_b (Ls), kept in the workspace for step 6 ----
#pragma unroll
        for (int j = 0; j < 16; ++j) Ls[er * LDX + 16 * ec + j] = Zs[er * LDX + 16 * ec + j];
        lds_barrier();
        for (int tb = 0; tb < NT; ++tb) {
            {
                float* dst = rst + static_cast<int64_t>(tb) * M * D + er * D + 16 * ec;
#pragma unroll
                for (int j = 0; j < 16; j += 4)
                    *reinterpret_cast<float4*>(dst + j) =
                        make_float4(Ls[er * LDX + 16 * ec + j], Ls[er * LDX + 16 * ec + j + 1],
                                    Ls[er * LDX + 16 * ec + j + 2], Ls[er * LDX + 16 * ec + j + 3]);
            }
            {
                // a_ref (.) dY_b R_b^T (the rest of dQA'), slot block w, into KAs (free since step 4)
                const f4 x = mm<D, LDX, 1, 1, LDX>(zero4(), Ys + TL * tb * LDX, Ls + 16 * w * LDX, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    KAs[(TL * tb + t_lane + r) * LDX + 16 * w + lc] = ar_s[tb * M + 16 * w + lc] * x[r];
            }
            if (tb + 1 < NT) {
                lds_barrier();  // every read of R_b done
                // R_{b+1} = diag(A_end) R_b - W_b^T H_b: wave w takes slots 16 w .. 16 w + 15
                f4 x[DT] = {zero4(), zero4(), zero4(), zero4()};
                mm4<TL, 1, LDX, LDX, 1, 16>(x, Ws + TL * tb * LDX + 16 * w, Hs + TL * tb * LDX, lane);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int sl = 16 * w + t_lane + r;
                        const int o = sl * LDX + 16 * dt + lc;
                        Ls[o] = fmaf(ae_s[tb * M + sl], Ls[o], -x[dt][r]);
                    }
                lds_barrier();
            }
        }
        lds_barrier();

        // ---- 6. tiles in reverse with lambda ----
        {
            const float* src = rst + static_cast<int64_t>(NT) * M * D + er * D + 16 * ec;
#pragma unroll
            for (int j = 0; j < 16; ++j) Ls[er * LDX + 16 * ec + j] = src[j];
        }
        lds_barrier();
        // R_b as this thread stored it, one tile ahead of its use
        float rb[16];
        {
            const float* src = rst + static_cast<int64_t>(NT - 1) * M * D + er * D + 16 * ec;
#pragma unroll
            for (int j = 0; j < 16; ++j) rb[j] = src[j];
        }
        for (int tb = NT - 1; tb >= 0; --tb) {
            {
                // dA_end = rowdot(R_b, lambda)
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 16; ++j) s = fmaf(rb[j], Ls[er * LDX + 16 * ec + j], s);
                s = quad_sum(s);
                if (ec == 0) dae_s[tb * M + er] = s;
                const float* src = rst + static_cast<int64_t>(tb > 0 ? tb - 1 : 0) * M * D + er * D + 16 * ec;
#pragma unroll
                for (int j = 0; j < 16; ++j) rb[j] = src[j];
            }
            // dW = -H_b lambda^T (slot block w) and dH_b -= W_b lambda (columns 16 w ..)
            const f4 dwx = mm<D, LDX, 1, 1, LDX>(zero4(), Hs + TL * tb * LDX, Ls + 16 * w * LDX, lane);
            {
                const f4 x = mm<M, LDX, 1, LDX, 1>(zero4(), Ws + TL * tb * LDX, Ls + 16 * w, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) Us[(TL * tb + t_lane + r) * LDX + 16 * w + lc] -= x[r];
            }
            lds_barrier();  // every read of lambda and of W_b done
            // dW over W_b in Ws (only step 7 reads it, as dW)
#pragma unroll
            for (int r = 0; r < 4; ++r) Ws[(TL * tb + t_lane + r) * LDX + 16 * w + lc] = -dwx[r];
            // lambda <- diag(A_end) lambda + a_ref (.) QA'^T dY_b: wave w takes slots 16 w ..
            {
                f4 x[DT] = {zero4(), zero4(), zero4(), zero4()};
                mm4<TL, 1, LDX, LDX, 1, 16>(x, QAs + TL * tb * LDX + 16 * w, Ys + TL * tb * LDX, lane);
#pragma unroll
                for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int sl = 16 * w + t_lane + r;
                        const int o = sl * LDX + 16 * dt + lc;
                        Ls[o] = fmaf(ae_s[tb * M + sl], Ls[o], ar_s[tb * M + sl] * x[dt][r]);
                    }
            }
            lds_barrier();
        }

        // ---- 7. per tile: gradients of A, W's suffix products, the gates ----
        float dht[MT][4], dkv[MT][4], dnh[4] = {0.f, 0.f, 0.f, 0.f}, dmu[4] = {0.f, 0.f, 0.f, 0.f};
        float dgt_tok[4] = {0.f, 0.f, 0.f, 0.f}, kqs[MT][4];
        float kq[4], qv[4], gm[4];  // slot block mt's inputs; block mt + 1's are loaded meanwhile
        load_in(0, kq, qv, gm);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            float kqn[4], qvn[4], gmn[4];
            load_in(mt + 1 < MT ? mt + 1 : mt, kqn, qvn, gmn);
            TileGates tg;
            tile_gates(kq, gm, mu, hh, ht[mt], lane, tg);
            const float dae = dae_s[w * M + 16 * mt + lc];
            float dA[4], dk_[4], u[4], X[4], Xp[4], dwt[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (TL * w + t_lane + r) * LDX + 16 * mt + lc;
                dqa[mt][r] += KAs[o];
                dwt[r] = Ws[o];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ka = tg.kap[r] * tg.ar * tg.rA[r];
                // dq = dQA' A / a_ref
                p.dq[bth(tc + t_lane + r) * M + 16 * mt + lc] = dqa[mt][r] * tg.A[r] * tg.rar;
                dA[r] = dqa[mt][r] * qv[r] * tg.rar - dka[mt][r] * ka * tg.rA[r];
                dk_[r] = dka[mt][r] * tg.ar * tg.rA[r] + dwt[r] * tg.sfx[r];
                u[r] = dwt[r] * tg.kap[r];
            }
            // the tile's last token: dA_end
            if (lg == 3) dA[3] += dae;
            // W_t = kappa_t prod_{l > t} g_l: dg_l += sfx_l sum_{s < l} dW_s kappa_s prod_{s < l' < l} g_l'
            affine_scan_fwd(tg.g, u, X, Xp, lane);
            float dg[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) dg[r] = Xp[r] * tg.sfx[r];
            // E_t = dA_t + g_{t+1} E_{t+1}; dg_t += A_{t-1} E_t
            float gn[4], E[4];
#pragma unroll
            for (int r = 0; r < 3; ++r) gn[r] = tg.g[r + 1];
            {
                // g of the next lane group's first token
                const float nx = __shfl(tg.g[0], (lc + 16 * (lg + 1)) & 63, 64);
                gn[3] = lg < 3 ? nx : 0.f;
            }
            affine_scan_rev(gn, dA, E, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) dg[r] = fmaf(tg.Ap[r], E[r], dg[r]);
            // through beta, kappa and g
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float a = tg.a[r], bt_ = tg.beta[r], wv = tg.wv[r];
                const bool msk = hh[r] - ht[mt][r] * ht[mt][r] > 0.f;
                const float dbeta = dg[r] * (mu[r] + a * ht[mt][r]) + dk_[r] * a;
                float dc = dg[r] * tg.kap[r];
                float da = dg[r] * bt_ * ht[mt][r] + dk_[r] * bt_;
                const float tb_ = -0.5f * bt_ * bt_ * bt_ * dbeta;
                dmu[r] += dg[r] * bt_ + 2.f * mu[r] * tb_;
                da = fmaf(2.f * a * wv, tb_, da);
                const float dw = msk ? a * a * tb_ : 0.f;
                dnh[r] += dw;
                dc -= 2.f * ht[mt][r] * dw;
                dht[mt][r] = dc;
                const float dgam = da * kq[r];
                if (gps)
                    p.dgamma[bth(tc + t_lane + r) * M + 16 * mt + lc] = dgam;
                else
                    dgt_tok[r] += dgam;
                dkv[mt][r] = da * gm[r];
                kqs[mt][r] = kq[r];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                kq[r] = kqn[r];
                qv[r] = qvn[r];
                gm[r] = gmn[r];
            }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            dnh[r] = row16_sum(dnh[r]);
            dmu[r] = row16_sum(dmu[r]);
            if (!gps) dgt_tok[r] = row16_sum(dgt_tok[r]);
        }
        if (lc == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t tt = bth(tc + t_lane + r);
                p.dmu[tt] = dmu[r];
                if (!gps) p.dgamma[tt] = dgt_tok[r];
                dnh_s[TL * w + t_lane + r] = dnh[r];
            }
        }
        // dc into QAs (token-major), K into KAs (decoding objective: K^T dH)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (TL * w + t_lane + r) * LDX + 16 * mt + lc;
                QAs[o] = dht[mt][r];
                KAs[o] = kqs[mt][r];
            }
        lds_barrier();

        // ---- 8. dH += dc Z + 2 d|h|^2 H; dV = -dH ----
        {
            f4 acc[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[dt][r] = Us[(TL * w + t_lane + r) * LDX + 16 * dt + lc];
            mm4<M, LDX, 1, LDX, 1, 16>(acc, QAs + TL * w * LDX, Zs, lane);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = TL * w + t_lane + r;
                    const float v = fmaf(2.f * dnh_s[t], Hs[t * LDX + 16 * dt + lc], acc[dt][r]);
                    Us[t * LDX + 16 * dt + lc] = v;
                    p.dv[bth(n * C + t) * D + 16 * dt + lc] = -v;
                }
        }
        lds_barrier();

        // ---- 9. dZ = lambda + dc^T H (+ K^T dH); dK = da gamma (+ dH Z^T) ----
        {
            f4 acc[DT];
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[dt][r] = Ls[(16 * w + t_lane + r) * LDX + 16 * dt + lc];
            mm4<C, 1, LDX, LDX, 1, 16>(acc, QAs + 16 * w, Hs, lane);
            if (dec) mm4<C, 1, LDX, LDX, 1, 16>(acc, KAs + 16 * w, Us, lane);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt)
#pragma unroll
                for (int r = 0; r < 4; ++r) Ls[(16 * w + t_lane + r) * LDX + 16 * dt + lc] = acc[dt][r];
        }
        {
            f4 acc[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[mt][r] = dkv[mt][r];
            if (dec) mm4<D, LDX, 1, 1, LDX, 16 * LDX>(acc, Us + TL * w * LDX, Zs, lane);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int r = 0; r < 4; ++r) p.dk[bth(tc + t_lane + r) * M + 16 * mt + lc] = acc[mt][r];
        }
        lds_barrier();

        // ---- 10. back through the chunk-start projection ----
        {
            float dz[16], zz[16], pr = 0.f;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                dz[j] = Ls[er * LDX + 16 * ec + j];
                zz[j] = Zs[er * LDX + 16 * ec + j];
                pr = fmaf(zz[j], dz[j], pr);
            }
            pr = quad_sum(pr);
            const float inv = invn_s[er];
            float* dst = rst + static_cast<int64_t>(NT) * M * D + er * D + 16 * ec;
#pragma unroll
            for (int j = 0; j < 16; ++j) dst[j] = inv * fmaf(-pr, zz[j], dz[j]);
        }
        lds_barrier();  // the next chunk overwrites every LDS array
    }
    {
        const float* src = rst + static_cast<int64_t>(NT) * M * D + er * D + 16 * ec;
        float* dst = p.dstate_in + static_cast<int64_t>(bh) * M * D + er * D + 16 * ec;
#pragma unroll
        for (int j = 0; j < 16; ++j) dst[j] = src[j];
    }
}

}  // namespace cbwd

// The chunk-form backward where it is built (m = d = C = 64, bf16 inputs, the
// default linearisation, decoding or similarity objective, chunk-start states
// from the state-passing kernel); -3 elsewhere.
bool bwd_chunk_supported(int m, int d, int C, bool in_bf16, bool lin1, int mode) {
    return m == 64 && d == 64 && C == 64 && in_bf16 && !lin1 && (mode == 0 || mode == 1);
}

int launch_bwd_chunk(int m, int d, const BwdParams& p, bool in_bf16, hipStream_t st) {
    if (!bwd_chunk_supported(m, d, p.f.chunk, in_bf16, p.f.lin1 != 0, p.f.mode) || !p.states_ready) return -3;
    const dim3 grid(static_cast<unsigned>(p.f.B) * static_cast<unsigned>(p.f.H));
    if (p.dy_bf16)
        hipLaunchKernelGGL((cbwd::osr_bwd_chunk_kernel<64, 64, 64, uint16_t, true>), grid, dim3(256), 0, st, p);
    else
        hipLaunchKernelGGL((cbwd::osr_bwd_chunk_kernel<64, 64, 64, uint16_t, false>), grid, dim3(256), 0, st, p);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace osr
