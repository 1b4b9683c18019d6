// osr_mfma_kernels.h -- chunk-wise OSR forward on gfx950 matrix cores.
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646), section "Parallel and Hardware Efficient Form".  Within a chunk
// every projection, gate and (decoding objective) h_t is taken at the
// unit-projected chunk-start state Z (eq. recurrence_linear2):
//   H      = K Z - V   (decoding)   or  -V   (similarity)       [C x d]
//   c      = H Z^T,  hh_t = |h_t|^2                             [C x m], [C]
//   a      = gamma (.) k,  w = max(hh - c^2, 0)
//   beta   = (mu^2 + a^2 w)^(-1/2)     (appendix "Computing beta", eq. beta_chunk)
//   g      = beta (mu + a c),  kappa = -beta a                  [C x m]
//   s_i   <- g_{t,i} s_i + kappa_{t,i} h_t,   y_t = sum_i q_{t,i} s_i
// which is a gated linear attention with keys kappa, values h, queries q and
// a per-key rank-one gate g.  The gated recurrence is evaluated in closed form
// over sub-blocks of C0 tokens (C0 = 16 or 32): with A the running product of
// g inside the sub-block and R the running state at its start,
//   Y   = (Q (.) A) R + tril[(Q (.) A)(kappa (/) A)^T] H
//   R  <- diag(A_end) R + W^T H,   W_t = kappa_t (.) prod_{l > t} g_l.
// Z and R are fp32; every product whose operand derives from the state runs
// as three bf16 MFMAs on a hi/lo split (hi*hi + hi*lo + lo*hi); k and q are
// exact bf16 inputs.
//
// Work layout: one workgroup of D/16 waves; wave w owns columns
// [16w, 16w + 16) of the state (as MFMA accumulators), of H and of Y.  With
// v_mfma_f32_16x16x16_bf16 an accumulator tile (lane l holds rows
// 4(l/16)+r of column l%16) is directly a B operand whose k index is the
// tile's row, so R feeds the read-out and H feeds the causal product and the
// state update without a transpose.  Contractions over d (c = H Z^T) and all
// A operands go through LDS.
#pragma once

#include "osr_device.h"

namespace osr {
namespace mfma {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mma(s16x4 a, s16x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// a*b with both operands split into bf16 hi + lo: the three significant terms,
// smallest first.
__device__ __forceinline__ f32x4 mma3(s16x4 ah, s16x4 al, s16x4 bh, s16x4 bl, f32x4 c) {
    c = mma(al, bh, c);
    c = mma(ah, bl, c);
    return mma(ah, bh, c);
}

__device__ __forceinline__ short bf16_bits(float x) {
    return __builtin_bit_cast(short, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_val(short b) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(b)) << 16);
}

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi).
__device__ __forceinline__ void split1(float x, short& hi, short& lo) {
    hi = bf16_bits(x);
    lo = bf16_bits(x - bf16_val(hi));
}
__device__ __forceinline__ void split4(f32x4 x, s16x4& hi, s16x4& lo) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        short h, l;
        split1(x[j], h, l);
        hi[j] = h;
        lo[j] = l;
    }
}

template <int M, int D, int C0>
struct Cfg {
    static constexpr int NW = D / 16;   // waves; wave w owns d-block w
    static constexpr int NT = 64 * NW;
    static constexpr int MT = M / 16;   // slot tiles
    static constexpr int TB = C0 / 16;  // token tiles per sub-block
    static constexpr int PAD = 8;       // bf16 elements of row padding
    static constexpr int ZS_LD = D + PAD;
    static constexpr int KS_LD = M + PAD;
    static constexpr int HS_LD = D + PAD;
    static constexpr int QA_LD = M + PAD;
    static constexpr int WT_LD = C0 + PAD;
    // Scalar (gate) phase: each slot column is split into NSEG token segments
    // of L tokens; SPT slots per thread when there are fewer threads than slots.
    static constexpr int SPT = M > NT ? M / NT : 1;
    static constexpr int NSEG0 = NT > M ? NT / M : 1;
    static constexpr int NSEG = NSEG0 < C0 ? NSEG0 : C0;
    static constexpr int L = C0 / NSEG;
    static constexpr int SCAL_THREADS = (M < NT ? M : NT) * NSEG;

    // LDS layout (bytes).
    static constexpr int O_ZH = 0;
    static constexpr int O_ZL = O_ZH + M * ZS_LD * 2;
    static constexpr int O_KS = O_ZL + M * ZS_LD * 2;
    static constexpr int O_HH = O_KS + C0 * KS_LD * 2;
    static constexpr int O_HL = O_HH + C0 * HS_LD * 2;
    static constexpr int O_CS = O_HL + C0 * HS_LD * 2;
    static constexpr int O_HP = O_CS + C0 * M * 4;           // hh partials [NW][C0]
    static constexpr int O_QH = O_HP + NW * C0 * 4;
    static constexpr int O_QL = O_QH + C0 * QA_LD * 2;
    static constexpr int O_KH = O_QL + C0 * QA_LD * 2;
    static constexpr int O_KL = O_KH + C0 * QA_LD * 2;
    static constexpr int O_WH = O_KL + C0 * QA_LD * 2;
    static constexpr int O_WL = O_WH + M * WT_LD * 2;
    static constexpr int O_AE = O_WL + M * WT_LD * 2;        // A_end [M]
    static constexpr int O_SG = O_AE + M * 4;                // segment products [NSEG][M]
    static constexpr int O_NP = O_SG + NSEG * M * 4;         // norm partials [NW][M]
    static constexpr int BYTES = O_NP + NW * M * 4;

    static_assert(M % 16 == 0 && D % 16 == 0 && C0 % 16 == 0, "tile multiples");
    static_assert(NW >= 1 && NT <= 1024, "waves");
    static_assert(L * NSEG == C0, "segments divide the sub-block");
    static_assert(SPT * NT >= M || M <= NT, "slots covered");
};

// LDS fits in one workgroup (160 KiB on gfx950).
template <int M, int D, int C0>
constexpr bool fits() {
    return Cfg<M, D, C0>::BYTES <= 160 * 1024;
}

// --------------------------------------------------------------------------
// One chunk for one (b, h).  acc_R holds the chunk-start state (projected by
// the caller); on return it holds the pre-projection state at the chunk end.
// WITH_Y: also form and store the read-outs y.
// need_state: also apply the update after the last sub-block.
template <int M, int D, int C0, bool WITH_Y>
__device__ __forceinline__ void osr_chunk(const Params& p, char* smem, f32x4 (&acc_R)[M / 16],
                                          int b, int hd, int t_chunk0, int C, bool need_state) {
    using G = Cfg<M, D, C0>;
    constexpr int MT = G::MT, TB = G::TB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lg = lane >> 4, lc = lane & 15;   // lane group (row quad) and column
    const int dcol = 16 * w + lc;               // this lane's state/H/Y column

    short* zh = reinterpret_cast<short*>(smem + G::O_ZH);
    short* zl = reinterpret_cast<short*>(smem + G::O_ZL);
    short* ks = reinterpret_cast<short*>(smem + G::O_KS);
    short* hsh = reinterpret_cast<short*>(smem + G::O_HH);
    short* hsl = reinterpret_cast<short*>(smem + G::O_HL);
    float* cs = reinterpret_cast<float*>(smem + G::O_CS);
    float* hp = reinterpret_cast<float*>(smem + G::O_HP);
    short* qah = reinterpret_cast<short*>(smem + G::O_QH);
    short* qal = reinterpret_cast<short*>(smem + G::O_QL);
    short* kah = reinterpret_cast<short*>(smem + G::O_KH);
    short* kal = reinterpret_cast<short*>(smem + G::O_KL);
    short* wth = reinterpret_cast<short*>(smem + G::O_WH);
    short* wtl = reinterpret_cast<short*>(smem + G::O_WL);
    float* aend = reinterpret_cast<float*>(smem + G::O_AE);
    float* segp = reinterpret_cast<float*>(smem + G::O_SG);

    const uint16_t* qg = static_cast<const uint16_t*>(p.q);
    const uint16_t* kg = static_cast<const uint16_t*>(p.k);
    const uint16_t* vg = static_cast<const uint16_t*>(p.v);
    const uint16_t* gg = static_cast<const uint16_t*>(p.gamma);
    const uint16_t* mug = static_cast<const uint16_t*>(p.mu);
    auto bth = [&](int t) { return (static_cast<int64_t>(b) * p.T + t) * p.H + hd; };

    // Z as B operands (k = slot) for H = K Z, and row-major in LDS for c = H Z^T.
    s16x4 zfh[MT], zfl[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        split4(acc_R[mt], zfh[mt], zfl[mt]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * lg + r;
            zh[row * G::ZS_LD + dcol] = zfh[mt][r];
            zl[row * G::ZS_LD + dcol] = zfl[mt][r];
        }
    }

    for (int u = 0; u < C; u += C0) {
        const int t0 = t_chunk0 + u;
        // ---- stage K of the sub-block (exact bf16) -------------------------
        for (int e = tid; e < C0 * M / 8; e += G::NT) {
            const int tau = e / (M / 8), i0 = (e % (M / 8)) * 8;
            const uint4 val = *reinterpret_cast<const uint4*>(kg + bth(t0 + tau) * M + i0);
            *reinterpret_cast<uint4*>(ks + tau * G::KS_LD + i0) = val;
        }
        __syncthreads();  // ks, and (first sub-block) zh/zl, visible

        // ---- H = K Z - V for this wave's columns ---------------------------
        f32x4 accH[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
            if (p.mode == 0) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const s16x4 kf = *reinterpret_cast<const s16x4*>(
                        ks + (16 * tb + lc) * G::KS_LD + 16 * mt + 4 * lg);
                    a = mma(kf, zfl[mt], a);
                    a = mma(kf, zfh[mt], a);
                }
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                a[r] -= bf16_bits_to_f32(vg[bth(t0 + 16 * tb + 4 * lg + r) * D + dcol]);
            accH[tb] = a;
        }
        // |h_t|^2 partial over this wave's columns; H row-major (hi/lo) to LDS.
        s16x4 hfh[TB], hfl[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            split4(accH[tb], hfh[tb], hfl[tb]);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int row = 16 * tb + 4 * lg + r;
                hsh[row * G::HS_LD + dcol] = hfh[tb][r];
                hsl[row * G::HS_LD + dcol] = hfl[tb][r];
                float sq = accH[tb][r] * accH[tb][r];
                sq = group_sum<16>(sq);
                if (lc == 0) hp[w * C0 + row] = sq;
            }
        }
        __syncthreads();  // H and |h|^2 partials visible

        // ---- c = H Z^T (contraction over all d), tiles spread over waves ---
        for (int ti = w; ti < TB * MT; ti += G::NW) {
            const int tb = ti / MT, mb = ti % MT;
            f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kd = 0; kd < D / 16; ++kd) {
                const int ao = (16 * tb + lc) * G::HS_LD + 16 * kd + 4 * lg;
                const int bo = (16 * mb + lc) * G::ZS_LD + 16 * kd + 4 * lg;
                a = mma3(*reinterpret_cast<const s16x4*>(hsh + ao), *reinterpret_cast<const s16x4*>(hsl + ao),
                         *reinterpret_cast<const s16x4*>(zh + bo), *reinterpret_cast<const s16x4*>(zl + bo), a);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r) cs[(16 * tb + 4 * lg + r) * M + 16 * mb + lc] = a[r];
        }
        __syncthreads();  // c visible

        // ---- gates: beta, g, kappa; running products along the sub-block ---
        // Pass 1: per (slot, token segment) the gates and the segment product.
        const bool sact = tid < G::SCAL_THREADS;
        float gt[G::SPT][G::L], kp[G::SPT][G::L];
        if (sact) {
#pragma unroll
            for (int sp = 0; sp < G::SPT; ++sp) {
                const int i = (G::SPT > 1) ? tid + sp * G::NT : tid % M;
                const int seg = (G::SPT > 1) ? 0 : tid / M;
                float run = 1.f;
#pragma unroll
                for (int j = 0; j < G::L; ++j) {
                    const int tau = seg * G::L + j;
                    const int64_t n = bth(t0 + tau);
                    float hh = 0.f;
#pragma unroll
                    for (int ww = 0; ww < G::NW; ++ww) hh += hp[ww * C0 + tau];
                    const float c = cs[tau * M + i];
                    const float k = bf16_val(ks[tau * G::KS_LD + i]);
                    const float gam = bf16_bits_to_f32(p.gamma_per_slot ? gg[n * M + i] : gg[n]);
                    const float mu = bf16_bits_to_f32(mug[n]);
                    const float a = gam * k;
                    const float wv = fmaxf(fmaf(-c, c, hh), 0.f);
                    const float beta = rsqrtf(fmaf(mu, mu, a * a * wv));
                    gt[sp][j] = beta * fmaf(a, c, mu);
                    kp[sp][j] = -beta * a;
                    run *= gt[sp][j];
                }
                segp[seg * M + i] = run;
            }
        }
        __syncthreads();  // segment products visible
        // Pass 2: running products A, suffix products, and the operands
        // Q (.) A, kappa (/) A (read-out) and W^T (state update).
        if (sact) {
#pragma unroll
            for (int sp = 0; sp < G::SPT; ++sp) {
                const int i = (G::SPT > 1) ? tid + sp * G::NT : tid % M;
                const int seg = (G::SPT > 1) ? 0 : tid / M;
                float before = 1.f, after = 1.f;
#pragma unroll
                for (int s2 = 0; s2 < G::NSEG; ++s2) {
                    const float v = segp[s2 * M + i];
                    if (s2 < seg) before *= v;
                    if (s2 > seg) after *= v;
                }
                float suf[G::L];
                float sacc = after;
#pragma unroll
                for (int j = G::L - 1; j >= 0; --j) {
                    suf[j] = sacc;
                    sacc *= gt[sp][j];
                }
                if (seg == 0) aend[i] = sacc;  // product over the whole sub-block
                float A = before;
#pragma unroll
                for (int j = 0; j < G::L; ++j) {
                    const int tau = seg * G::L + j;
                    A *= gt[sp][j];
                    short hi, lo;
                    split1(kp[sp][j] * suf[j], hi, lo);
                    wth[i * G::WT_LD + tau] = hi;
                    wtl[i * G::WT_LD + tau] = lo;
                    if constexpr (WITH_Y) {
                        const float q = bf16_bits_to_f32(qg[bth(t0 + tau) * M + i]);
                        split1(q * A, hi, lo);
                        qah[tau * G::QA_LD + i] = hi;
                        qal[tau * G::QA_LD + i] = lo;
                        split1(kp[sp][j] / A, hi, lo);
                        kah[tau * G::QA_LD + i] = hi;
                        kal[tau * G::QA_LD + i] = lo;
                    }
                }
            }
        }
        __syncthreads();  // W^T, A_end (and Q.A, kappa/A) visible

        // ---- read-out: Y = (Q.A) R + tril(P) H, P^T = (kappa/A)(Q.A)^T ---
        if constexpr (WITH_Y) {
            s16x4 rfh[MT], rfl[MT];
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (u == 0) {
                    rfh[mt] = zfh[mt];
                    rfl[mt] = zfl[mt];
                } else {
                    split4(acc_R[mt], rfh[mt], rfl[mt]);
                }
            }
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                f32x4 y = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int ao = (16 * tb + lc) * G::QA_LD + 16 * mt + 4 * lg;
                    y = mma3(*reinterpret_cast<const s16x4*>(qah + ao), *reinterpret_cast<const s16x4*>(qal + ao),
                             rfh[mt], rfl[mt], y);
                }
#pragma unroll
                for (int jb = 0; jb <= tb; ++jb) {
                    f32x4 pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int ao = (16 * jb + lc) * G::QA_LD + 16 * mt + 4 * lg;
                        const int bo = (16 * tb + lc) * G::QA_LD + 16 * mt + 4 * lg;
                        pt = mma3(*reinterpret_cast<const s16x4*>(kah + ao), *reinterpret_cast<const s16x4*>(kal + ao),
                                  *reinterpret_cast<const s16x4*>(qah + bo), *reinterpret_cast<const s16x4*>(qal + bo), pt);
                    }
                    if (jb == tb) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * lg + r > lc) pt[r] = 0.f;  // causal: j <= tau
                    }
                    s16x4 ph, pl;
                    split4(pt, ph, pl);
                    y = mma3(ph, pl, hfh[jb], hfl[jb], y);
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    st_y1(p.y, bth(t0 + 16 * tb + 4 * lg + r) * D + dcol, y[r], p.y_bf16);
            }
        }

        // ---- state update: R <- diag(A_end) R + W^T H ----------------------
        if (need_state || u + C0 < C) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                f32x4 a = acc_R[mt];
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] *= aend[16 * mt + 4 * lg + r];
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int ao = (16 * mt + lc) * G::WT_LD + 16 * tb + 4 * lg;
                    a = mma3(*reinterpret_cast<const s16x4*>(wth + ao), *reinterpret_cast<const s16x4*>(wtl + ao),
                             hfh[tb], hfl[tb], a);
                }
                acc_R[mt] = a;
            }
        }
    }
}

// Project every slot (row) of the accumulator-held state onto the unit
// sphere: sums of squares over each wave's 16 columns, then across waves.
template <int M, int D, int C0>
__device__ __forceinline__ void project_state(f32x4 (&acc)[M / 16], char* smem) {
    using G = Cfg<M, D, C0>;
    float* np = reinterpret_cast<float*>(smem + G::O_NP);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, lc = lane & 15;
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float s = group_sum<16>(acc[mt][r] * acc[mt][r]);
            if (lc == 0) np[w * M + 16 * mt + 4 * lg + r] = s;
        }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < G::MT; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float n2 = 0.f;
#pragma unroll
            for (int ww = 0; ww < G::NW; ++ww) n2 += np[ww * M + 16 * mt + 4 * lg + r];
            acc[mt][r] *= rsqrtf(n2);
        }
    __syncthreads();
}

template <int M, int D>
__device__ __forceinline__ void load_rows(f32x4 (&acc)[M / 16], const float* src) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, lc = lane & 15;
#pragma unroll
    for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[mt][r] = src[(16 * mt + 4 * lg + r) * D + 16 * w + lc];
}

template <int M, int D>
__device__ __forceinline__ void store_rows(const f32x4 (&acc)[M / 16], float* dst) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, lc = lane & 15;
#pragma unroll
    for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) dst[(16 * mt + 4 * lg + r) * D + 16 * w + lc] = acc[mt][r];
}

// Sequential chunk loop for one (b, h) per workgroup.
//   WITH_Y = false, WRITE_Z = true : inter-chunk state-passing kernel; stores
//       every chunk-start state to p.zbuf for the intra-chunk kernel.
//   WITH_Y = true,  WRITE_Z = false: fused forward (state passing + read-out).
template <int M, int D, int C0, bool WITH_Y, bool WRITE_Z>
__global__ __launch_bounds__(4 * D) void osr_chunk_loop_kernel(Params p) {
    using G = Cfg<M, D, C0>;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    const int bh = blockIdx.x, b = bh / p.H, hd = bh % p.H;
    const int C = p.chunk, NC = p.T / C;
    f32x4 acc[G::MT];
    load_rows<M, D>(acc, p.state_in + static_cast<int64_t>(bh) * M * D);
    for (int ch = 0; ch < NC; ++ch) {
        project_state<M, D, C0>(acc, smem);
        if constexpr (WRITE_Z)
            store_rows<M, D>(acc, p.zbuf + (static_cast<int64_t>(bh) * NC + ch) * M * D);
        osr_chunk<M, D, C0, WITH_Y>(p, smem, acc, b, hd, ch * C, C, true);
    }
    project_state<M, D, C0>(acc, smem);
    store_rows<M, D>(acc, p.state_out + static_cast<int64_t>(bh) * M * D);
}

// Intra-chunk read-out: one workgroup per (chunk, b, h), starting from the
// chunk-start state the state-passing kernel stored.
template <int M, int D, int C0>
__global__ __launch_bounds__(4 * D) void osr_intra_chunk_kernel(Params p) {
    using G = Cfg<M, D, C0>;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    const int BH = p.B * p.H, C = p.chunk, NC = p.T / C;
    const int ch = blockIdx.x / BH, bh = blockIdx.x % BH;
    const int b = bh / p.H, hd = bh % p.H;
    f32x4 acc[G::MT];
    load_rows<M, D>(acc, p.zbuf + (static_cast<int64_t>(bh) * NC + ch) * M * D);
    osr_chunk<M, D, C0, true>(p, smem, acc, b, hd, ch * C, C, false);
}

}  // namespace mfma
}  // namespace osr
