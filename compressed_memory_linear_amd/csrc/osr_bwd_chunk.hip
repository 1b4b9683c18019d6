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
// throughout).  Eight waves: wave w takes tile w & 3 and half w >> 2, whose
// per-(token, slot) values (slot blocks 2 half, 2 half + 1) live in its
// registers in the accumulator layout (lane (lg, lc) holds tokens 4lg..4lg+3
// of slot column lc of a 16-slot block).  The chunk-start states come from
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
#pragma unroll 8
    for (int k0 = 0; k0 < K; k0 += 4) acc = __builtin_amdgcn_mfma_f32_16x16x4f32(pa[k0 * AK], pb[k0 * BK], acc, 0, 0, 0);
    return acc;
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

// Two output tiles that share the A operand (acc[j] += A B_j, B_j at b + j * BS).
template <int K, int AI, int AK, int BK, int BJ, int BS>
__device__ __forceinline__ void mm2(f4 (&acc)[2], const float* a, const float* b, int lane) {
    const int r = lane & 15, kq = lane >> 4;
    const float* pa = a + r * AI + kq * AK;
    const float* pb = b + kq * BK + r * BJ;
#pragma unroll 8
    for (int k0 = 0; k0 < K; k0 += 4) {
        const float av = pa[k0 * AK];
        const float b0 = pb[k0 * BK], b1 = pb[k0 * BK + BS];
        acc[0] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b0, acc[0], 0, 0, 0);
        acc[1] = __builtin_amdgcn_mfma_f32_16x16x4f32(av, b1, acc[1], 0, 0, 0);
    }
}

// Sum over the 8 consecutive lanes of an element row (the M x D passes).
__device__ __forceinline__ float oct_sum(float x) {
    x += __shfl_xor(x, 1, 64);
    x += __shfl_xor(x, 2, 64);
    x += __shfl_xor(x, 4, 64);
    return x;
}

template <int M, int D, int C, typename TIn, bool DYB>
struct Cfg {
    static constexpr int LDX = 68;  // row stride (floats) of the LDS matrices
    static constexpr int NT = C / TL;
    static constexpr int MT = M / 16, DT = D / 16;
    static constexpr int NWAVE = 8;  // waves (b, hf): tile b = w & 3, half hf = w >> 2
    static constexpr int NTH = 64 * NWAVE;
    static_assert(M == 64 && D == 64 && C == 64, "built for m = d = C = 64");
    static_assert(NT == 4 && MT == 4 && DT == 4, "4 tiles, 4 slot blocks, 4 column blocks");
};

template <int M, int D, int C, typename TIn, bool DYB>
__global__ __launch_bounds__(512) void osr_bwd_chunk_kernel(BwdParams p) {
    using G = Cfg<M, D, C, TIn, DYB>;
    constexpr int LDX = G::LDX, NT = G::NT;
    __shared__ __attribute__((aligned(16))) float Zs[M * LDX];   // Z
    __shared__ __attribute__((aligned(16))) float Hs[C * LDX];   // H
    __shared__ __attribute__((aligned(16))) float Ys[C * LDX];   // dY
    __shared__ __attribute__((aligned(16))) float Us[C * LDX];   // V, then dH
    __shared__ __attribute__((aligned(16))) float Ls[M * LDX];   // R_b, then lambda, then dZ
    __shared__ __attribute__((aligned(16))) float QAs[C * LDX];  // Q A / a_ref, then dc
    __shared__ __attribute__((aligned(16))) float KAs[C * LDX];  // kappa a_ref / A, then dQA' parts, then K
    __shared__ __attribute__((aligned(16))) float Ws[C * LDX];   // K, then W, then dW
    __shared__ float Ps[NT][16 * 17], dPs[NT][16 * 17];          // per tile: P, dP ([t][u])
    __shared__ float part_s[2][3][C];  // per-token sums of the two halves: |h|^2, d|h|^2, dmu (and dgamma)
    __shared__ float pg_s[2][C];
    __shared__ float ae_s[NT * M], ar_s[NT * M], dae_s[NT * M], invn_s[M];

    const int bh = blockIdx.x, b = bh / p.f.H, hd = bh % p.f.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, lg = lane >> 4, lc = lane & 15;
    const int tw = w & 3, hf = w >> 2;  // this wave's tile and half (slot / column blocks 2 hf, 2 hf + 1)
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
    float* rst = ws + static_cast<int64_t>(NC + 1) * M * D;     // [NT][M][D] tile-start states, then lambda
    auto bth = [&](int t) { return (static_cast<int64_t>(b) * T + t) * p.f.H + hd; };

    // M x D element passes: row er, columns 8 ec .. 8 ec + 7
    const int er = tid >> 3, ec = tid & 7;
    const int eo = er * LDX + 8 * ec, go = er * D + 8 * ec;

    {
        // the returned state is the end state projected: its backward; lambda lives in the
        // workspace between chunks (each thread its own elements)
        const float* s = sck + static_cast<int64_t>(NC) * M * D + go;
        const float* g = p.dstate_out + static_cast<int64_t>(bh) * M * D + go;
        float sv[8], lv[8], n2 = 0.f, pr = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            sv[j] = s[j];
            lv[j] = g[j];
            n2 += sv[j] * sv[j];
        }
        const float inv = rsqrtf(oct_sum(n2));
#pragma unroll
        for (int j = 0; j < 8; ++j) pr += sv[j] * inv * lv[j];
        pr = oct_sum(pr);
        float* dst = rst + static_cast<int64_t>(NT) * M * D + go;
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[j] = inv * (lv[j] - pr * sv[j] * inv);
    }
    const int t_lane = 4 * lg;  // first token (within the tile) of this lane's rows
    for (int n = NC - 1; n >= 0; --n) {
        const int tc = n * C + TL * tw;  // first token of this wave's tile
        // ---- 1. Z, V, dY, K into LDS; this tile's mu ----
        {
            const float* s = sck + static_cast<int64_t>(n) * M * D + go;
            float sv[8], n2 = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                sv[j] = s[j];
                n2 += sv[j] * sv[j];
            }
            const float inv = rsqrtf(oct_sum(n2));
#pragma unroll
            for (int j = 0; j < 8; ++j) Zs[eo + j] = sv[j] * inv;
            if (ec == 0) invn_s[er] = inv;
            // token rows: V and dY [C][D], K [C][M] (er is the token here)
            const int64_t tv = bth(n * C + er);
#pragma unroll
            for (int j = 0; j < 8; j += 4) {
                const float4 v4 = ld4<TIn>(vp, tv * D + 8 * ec + j);
                float4 y4;
                if constexpr (DYB)
                    y4 = ld4<uint16_t>(static_cast<const uint16_t*>(p.dy), tv * D + 8 * ec + j);
                else
                    y4 = ld4<float>(static_cast<const float*>(p.dy), tv * D + 8 * ec + j);
                const float4 k4 = ld4<TIn>(kp, tv * M + 8 * ec + j);
                *reinterpret_cast<float4*>(Us + eo + j) = v4;
                *reinterpret_cast<float4*>(Ys + eo + j) = y4;
                *reinterpret_cast<float4*>(Ws + eo + j) = k4;
            }
        }
        float mu[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) mu[r] = ld<TIn>(mp, bth(tc + t_lane + r));
        // this wave's slot blocks 2 hf + j of its tile: k, q, gamma
        auto load_in = [&](int mt, float (&kq)[4], float (&qv)[4], float (&gm)[4]) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t tt = bth(tc + t_lane + r);
                kq[r] = ld<TIn>(kp, tt * M + 16 * mt + lc);
                qv[r] = ld<TIn>(qp, tt * M + 16 * mt + lc);
                gm[r] = gps ? ld<TIn>(gp, tt * M + 16 * mt + lc) : ld<TIn>(gp, tt);
            }
        };
        float kq3[2][4], qv3[2][4], gm3[2][4];
#pragma unroll
        for (int j = 0; j < 2; ++j) load_in(2 * hf + j, kq3[j], qv3[j], gm3[j]);
        lds_barrier();

        // ---- 2. H = K Z - V: tile tw, column blocks 2 hf, 2 hf + 1; |h|^2 ----
        float hh[4];
        {
            f4 acc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[j][r] = -Us[(TL * tw + t_lane + r) * LDX + 16 * (2 * hf + j) + lc];
            if (dec) mm2<M, LDX, 1, LDX, 1, 16>(acc, Ws + TL * tw * LDX, Zs + 32 * hf, lane);
            float ph[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    Hs[(TL * tw + t_lane + r) * LDX + 16 * (2 * hf + j) + lc] = acc[j][r];
                    ph[r] += acc[j][r] * acc[j][r];
                }
#pragma unroll
            for (int r = 0; r < 4; ++r) ph[r] = row16_sum(ph[r]);
            if (lc == 0)
#pragma unroll
                for (int r = 0; r < 4; ++r) part_s[hf][0][TL * tw + t_lane + r] = ph[r];
        }
        lds_barrier();  // H visible; every wave is done with K in Ws
#pragma unroll
        for (int r = 0; r < 4; ++r) hh[r] = part_s[0][0][TL * tw + t_lane + r] + part_s[1][0][TL * tw + t_lane + r];

        // ---- 3. c = H Z^T (tile tw, slot blocks 2 hf + j) and the gates ----
        float ht[2][4];
        {
            f4 acc[2] = {zero4(), zero4()};
            mm2<D, LDX, 1, 1, LDX, 16 * LDX>(acc, Hs + TL * tw * LDX, Zs + 32 * hf * LDX, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) ht[j][r] = acc[j][r];
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int mt = 2 * hf + j;
            TileGates tg;
            tile_gates(kq3[j], gm3[j], mu, hh, ht[j], lane, tg);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (TL * tw + t_lane + r) * LDX + 16 * mt + lc;
                QAs[o] = qv3[j][r] * tg.A[r] * tg.rar;
                KAs[o] = tg.kap[r] * tg.ar * tg.rA[r];
                Ws[o] = tg.kap[r] * tg.sfx[r];
            }
            if (lg == 0) {
                ae_s[tw * M + 16 * mt + lc] = tg.ae;
                ar_s[tw * M + 16 * mt + lc] = tg.ar;
            }
        }
        lds_barrier();

        // ---- 4. per tile: P (half 0), dP (half 1), then the lambda-free gradients ----
        {
            f4 x = zero4();
            if (hf == 0)
                x = mm<M, LDX, 1, 1, LDX>(x, QAs + TL * tw * LDX, KAs + TL * tw * LDX, lane);
            else
                x = mm<D, LDX, 1, 1, LDX>(x, Ys + TL * tw * LDX, Hs + TL * tw * LDX, lane);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const bool causal = lc <= t_lane + r;  // u <= t
                if (hf == 0)
                    Ps[tw][(t_lane + r) * 17 + lc] = causal ? x[r] : 0.f;
                else
                    dPs[tw][(t_lane + r) * 17 + lc] = causal ? -x[r] : 0.f;
            }
        }
        lds_barrier();
        float dqa[2][4], dka[2][4];  // (dqa goes to KAs at the next barrier)
        {
            // dQA' = dP KA', dKA' = dP^T QA' (slot blocks 2 hf + j), dH = -P^T dY (column blocks 2 hf + j,
            // into Us: V is dead since step 2)
            f4 x[2] = {zero4(), zero4()}, y[2] = {zero4(), zero4()}, z[2] = {zero4(), zero4()};
            mm2<TL, 17, 1, LDX, 1, 16>(x, dPs[tw], KAs + TL * tw * LDX + 32 * hf, lane);
            mm2<TL, 1, 17, LDX, 1, 16>(y, dPs[tw], QAs + TL * tw * LDX + 32 * hf, lane);
            mm2<TL, 1, 17, LDX, 1, 16>(z, Ps[tw], Ys + TL * tw * LDX + 32 * hf, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    dqa[j][r] = x[j][r];
                    dka[j][r] = y[j][r];
                    Us[(TL * tw + t_lane + r) * LDX + 16 * (2 * hf + j) + lc] = -z[j][r];
                }
        }

        // ---- 5. tile-start states R_b (Ls), kept in the workspace for step 6 ----
        lds_barrier();  // every read of KAs (as kappa a_ref / A) done: dQA' so far into it
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) KAs[(TL * tw + t_lane + r) * LDX + 16 * (2 * hf + j) + lc] = dqa[j][r];
        {
            float* dst = rst + go;
            const float4 z0 = *reinterpret_cast<const float4*>(Zs + eo);
            const float4 z1 = *reinterpret_cast<const float4*>(Zs + eo + 4);
            *reinterpret_cast<float4*>(Ls + eo) = z0;
            *reinterpret_cast<float4*>(Ls + eo + 4) = z1;
            *reinterpret_cast<float4*>(dst) = z0;
            *reinterpret_cast<float4*>(dst + 4) = z1;
        }
        lds_barrier();
        for (int tb = 0; tb < NT; ++tb) {
            if (hf == 0) {
                // a_ref (.) dY_b R_b^T (the rest of dQA'), slot block tw, into KAs
                const f4 x = mm<D, LDX, 1, 1, LDX>(zero4(), Ys + TL * tb * LDX, Ls + 16 * tw * LDX, lane);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    // (the tile's owner wrote its part of dQA' here before the barrier above)
                    const int o = (TL * tb + t_lane + r) * LDX + 16 * tw + lc;
                    KAs[o] = fmaf(ar_s[tb * M + 16 * tw + lc], x[r], KAs[o]);
                }
            }
            if (tb + 1 < NT) {
                lds_barrier();  // every read of R_b done
                // R_{b+1} = diag(A_end) R_b - W_b^T H_b: slot block tw, column blocks 2 hf + j
                f4 x[2] = {zero4(), zero4()};
                mm2<TL, 1, LDX, LDX, 1, 16>(x, Ws + TL * tb * LDX + 16 * tw, Hs + TL * tb * LDX + 32 * hf, lane);
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int sl = 16 * tw + t_lane + r;
                        const int o = sl * LDX + 16 * (2 * hf + j) + lc;
                        Ls[o] = fmaf(ae_s[tb * M + sl], Ls[o], -x[j][r]);
                    }
                lds_barrier();
                float* dst = rst + static_cast<int64_t>(tb + 1) * M * D + go;
                *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(Ls + eo);
                *reinterpret_cast<float4*>(dst + 4) = *reinterpret_cast<const float4*>(Ls + eo + 4);
            }
        }
        lds_barrier();

        // ---- 6. tiles in reverse with lambda ----
        {
            const float* src = rst + static_cast<int64_t>(NT) * M * D + go;
            *reinterpret_cast<float4*>(Ls + eo) = *reinterpret_cast<const float4*>(src);
            *reinterpret_cast<float4*>(Ls + eo + 4) = *reinterpret_cast<const float4*>(src + 4);
        }
        lds_barrier();
        // step 7's inputs again (not kept since step 3), loaded during the sweep
#pragma unroll
        for (int j = 0; j < 2; ++j) load_in(2 * hf + j, kq3[j], qv3[j], gm3[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) mu[r] = ld<TIn>(mp, bth(tc + t_lane + r));
        float rb[8];  // R_b as this thread stored it, one tile ahead of its use
        {
            const float* src = rst + static_cast<int64_t>(NT - 1) * M * D + go;
#pragma unroll
            for (int j = 0; j < 8; ++j) rb[j] = src[j];
        }
        for (int tb = NT - 1; tb >= 0; --tb) {
            {
                // dA_end = rowdot(R_b, lambda)
                float s = 0.f;
#pragma unroll
                for (int j = 0; j < 8; ++j) s = fmaf(rb[j], Ls[eo + j], s);
                s = oct_sum(s);
                if (ec == 0) dae_s[tb * M + er] = s;
                const float* src = rst + static_cast<int64_t>(tb > 0 ? tb - 1 : 0) * M * D + go;
#pragma unroll
                for (int j = 0; j < 8; ++j) rb[j] = src[j];
            }
            // half 0: dW = -H_b lambda^T (slot block tw); half 1: dH_b -= W_b lambda (column block tw)
            f4 x;
            if (hf == 0)
                x = mm<D, LDX, 1, 1, LDX>(zero4(), Hs + TL * tb * LDX, Ls + 16 * tw * LDX, lane);
            else
                x = mm<M, LDX, 1, LDX, 1>(zero4(), Ws + TL * tb * LDX, Ls + 16 * tw, lane);
            lds_barrier();  // every read of lambda and of W_b done
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (TL * tb + t_lane + r) * LDX + 16 * tw + lc;
                if (hf == 0)
                    Ws[o] = -x[r];  // dW over W_b (only step 7 reads it, as dW)
                else
                    Us[o] -= x[r];
            }
            // lambda <- diag(A_end) lambda + a_ref (.) QA'^T dY_b: slot block tw, column blocks 2 hf + j
            {
                f4 y[2] = {zero4(), zero4()};
                mm2<TL, 1, LDX, LDX, 1, 16>(y, QAs + TL * tb * LDX + 16 * tw, Ys + TL * tb * LDX + 32 * hf, lane);
#pragma unroll
                for (int j = 0; j < 2; ++j)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int sl = 16 * tw + t_lane + r;
                        const int o = sl * LDX + 16 * (2 * hf + j) + lc;
                        Ls[o] = fmaf(ae_s[tb * M + sl], Ls[o], ar_s[tb * M + sl] * y[j][r]);
                    }
            }
            lds_barrier();
        }

        // ---- 7. per tile and half: gradients of A, W's suffix products, the gates ----
        float dht[2][4], dkv[2][4], dnh[4] = {0.f, 0.f, 0.f, 0.f}, dmu[4] = {0.f, 0.f, 0.f, 0.f};
        float dgt_tok[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) hh[r] = part_s[0][0][TL * tw + t_lane + r] + part_s[1][0][TL * tw + t_lane + r];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int mt = 2 * hf + j;
            TileGates tg;
            tile_gates(kq3[j], gm3[j], mu, hh, ht[j], lane, tg);
            const float dae = dae_s[tw * M + 16 * mt + lc];
            float dA[4], dk_[4], u[4], X[4], Xp[4], dwt[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (TL * tw + t_lane + r) * LDX + 16 * mt + lc;
                dqa[j][r] = KAs[o];
                dwt[r] = Ws[o];
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float ka = tg.kap[r] * tg.ar * tg.rA[r];
                // dq = dQA' A / a_ref
                p.dq[bth(tc + t_lane + r) * M + 16 * mt + lc] = dqa[j][r] * tg.A[r] * tg.rar;
                dA[r] = dqa[j][r] * qv3[j][r] * tg.rar - dka[j][r] * ka * tg.rA[r];
                dk_[r] = dka[j][r] * tg.ar * tg.rA[r] + dwt[r] * tg.sfx[r];
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
                const bool msk = hh[r] - ht[j][r] * ht[j][r] > 0.f;
                const float dbeta = dg[r] * (mu[r] + a * ht[j][r]) + dk_[r] * a;
                float dc = dg[r] * tg.kap[r];
                float da = dg[r] * bt_ * ht[j][r] + dk_[r] * bt_;
                const float tb_ = -0.5f * bt_ * bt_ * bt_ * dbeta;
                dmu[r] += dg[r] * bt_ + 2.f * mu[r] * tb_;
                da = fmaf(2.f * a * wv, tb_, da);
                const float dw = msk ? a * a * tb_ : 0.f;
                dnh[r] += dw;
                dc -= 2.f * ht[j][r] * dw;
                dht[j][r] = dc;
                const float dgam = da * kq3[j][r];
                if (gps)
                    p.dgamma[bth(tc + t_lane + r) * M + 16 * mt + lc] = dgam;
                else
                    dgt_tok[r] += dgam;
                dkv[j][r] = da * gm3[j][r];
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
                const int t = TL * tw + t_lane + r;
                part_s[hf][1][t] = dnh[r];
                part_s[hf][2][t] = dmu[r];
                pg_s[hf][t] = dgt_tok[r];
            }
        }
        // dc into QAs (token-major), K into KAs (decoding objective: K^T dH)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int o = (TL * tw + t_lane + r) * LDX + 16 * (2 * hf + j) + lc;
                QAs[o] = dht[j][r];
                KAs[o] = kq3[j][r];
            }
        lds_barrier();
        if (hf == 0 && lc == 0) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int t = TL * tw + t_lane + r;
                const int64_t tt = bth(n * C + t);
                p.dmu[tt] = part_s[0][2][t] + part_s[1][2][t];
                if (!gps) p.dgamma[tt] = pg_s[0][t] + pg_s[1][t];
            }
        }

        // ---- 8. dH += dc Z + 2 d|h|^2 H (tile tw, column blocks 2 hf + j); dV = -dH ----
        {
            f4 acc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[j][r] = Us[(TL * tw + t_lane + r) * LDX + 16 * (2 * hf + j) + lc];
            mm2<M, LDX, 1, LDX, 1, 16>(acc, QAs + TL * tw * LDX, Zs + 32 * hf, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int t = TL * tw + t_lane + r, c = 16 * (2 * hf + j) + lc;
                    const float dn = part_s[0][1][t] + part_s[1][1][t];
                    const float v = fmaf(2.f * dn, Hs[t * LDX + c], acc[j][r]);
                    Us[t * LDX + c] = v;
                    p.dv[bth(n * C + t) * D + c] = -v;
                }
        }
        lds_barrier();

        // ---- 9. dZ = lambda + dc^T H (+ K^T dH) (slot block tw, column blocks 2 hf + j);
        //         dK = da gamma (+ dH Z^T) (tile tw, slot blocks 2 hf + j) ----
        {
            f4 acc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[j][r] = Ls[(16 * tw + t_lane + r) * LDX + 16 * (2 * hf + j) + lc];
            mm2<C, 1, LDX, LDX, 1, 16>(acc, QAs + 16 * tw, Hs + 32 * hf, lane);
            if (dec) mm2<C, 1, LDX, LDX, 1, 16>(acc, KAs + 16 * tw, Us + 32 * hf, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) Ls[(16 * tw + t_lane + r) * LDX + 16 * (2 * hf + j) + lc] = acc[j][r];
        }
        {
            f4 acc[2];
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[j][r] = dkv[j][r];
            if (dec) mm2<D, LDX, 1, 1, LDX, 16 * LDX>(acc, Us + TL * tw * LDX, Zs + 32 * hf * LDX, lane);
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) p.dk[bth(tc + t_lane + r) * M + 16 * (2 * hf + j) + lc] = acc[j][r];
        }
        lds_barrier();

        // ---- 10. back through the chunk-start projection ----
        {
            float dz[8], zz[8], pr = 0.f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                dz[j] = Ls[eo + j];
                zz[j] = Zs[eo + j];
                pr = fmaf(zz[j], dz[j], pr);
            }
            pr = oct_sum(pr);
            const float inv = invn_s[er];
            float* dst = rst + static_cast<int64_t>(NT) * M * D + go;
#pragma unroll
            for (int j = 0; j < 8; ++j) dst[j] = inv * fmaf(-pr, zz[j], dz[j]);
        }
        lds_barrier();  // the next chunk overwrites every LDS array
    }
    {
        const float* src = rst + static_cast<int64_t>(NT) * M * D + go;
        float* dst = p.dstate_in + static_cast<int64_t>(bh) * M * D + go;
#pragma unroll
        for (int j = 0; j < 8; ++j) dst[j] = src[j];
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
        hipLaunchKernelGGL((cbwd::osr_bwd_chunk_kernel<64, 64, 64, uint16_t, true>), grid, dim3(512), 0, st, p);
    else
        hipLaunchKernelGGL((cbwd::osr_bwd_chunk_kernel<64, 64, 64, uint16_t, false>), grid, dim3(512), 0, st, p);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace osr
