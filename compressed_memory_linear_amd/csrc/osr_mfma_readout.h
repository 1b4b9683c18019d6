// osr_mfma_readout.h -- read-out of the chunk-wise OSR forward on gfx950
// matrix cores, in parallel over chunks.
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646), section "Parallel and Hardware Efficient Form", eq.
// recurrence_linear2 and its gated-linear-attention form.  Inside a chunk the
// state evolves as s_i <- g_{t,i} s_i + kappa_{t,i} h_t with gates and h_t
// taken at the chunk-start state Z; the read-out is y_t = sum_i q_{t,i} s_i.
// The state-passing kernel stores, per chunk, Z, g, kappa and h (workspace,
// the per-token values in MFMA lane order);
// here each workgroup takes cpw consecutive chunks of one (b, h) and, over
// sub-blocks of C0 tokens with R the state at the sub-block start and A the
// running product of g inside the sub-block,
//   Y  = (Q (.) A) R + tril[(Q (.) A)(kappa (/) A)^T] H
//   R <- diag(A_end) R + W^T H,   W_t = kappa_t (.) prod_{l > t} g_l.
// R starts at Z for every chunk.  Products whose operands derive from the
// state, the gates or h run as three bf16 MFMAs on a hi/lo split.
//
// Work layout: D/16 waves; wave w owns columns [16w, 16w + 16) of R, H and Y
// (R as MFMA accumulator tiles, which are B operands with k = slot).  The
// per-(token, slot) gate products are formed by the wave that owns the slot
// block, which writes Q.A, kappa/A (token-major) and W^T (slot-major) to
// LDS; the causal tiles P are formed once and shared through LDS; two
// barriers per sub-block (the LDS buffers alternate between sub-blocks).
// All global inputs of sub-block s+1 are loaded into registers while s
// computes.
#pragma once

#include "osr_mfma_kernels.h"

namespace osr {
namespace mfma {

template <int M, int D, int C0, bool LIN1 = false>
struct ReadCfg {
    static constexpr bool LIN1_ = LIN1;
    static constexpr int NW = D / 16;  // wave w owns columns [16w, 16w + 16)
    static constexpr int NT = 64 * NW;
    static constexpr int MT = M / 16;
    static constexpr int TB = C0 / 16;
    static constexpr int MPW = (MT + NW - 1) / NW;  // slot tiles per wave in the gate phase
    // Row strides (bf16 elements): 8-byte operand reads of 16 rows and
    // scattered 2-byte writes of rows 4lg + r are conflict-free with a stride
    // of 2 (mod 4) words.
    static constexpr int QA_LD = M + 4;
    static constexpr int WT_LD = C0 + 4;
    static constexpr bool K32_C = C0 % 32 == 0; // R += W^T H          (k = token)
    // One LDS buffer set (bytes); two sets alternate between sub-blocks.
    static constexpr int B_QH = 0;                       // Q.A hi      [C0][QA_LD]
    static constexpr int B_QL = B_QH + C0 * QA_LD * 2;   // Q.A lo
    static constexpr int B_KH = B_QL + C0 * QA_LD * 2;   // kappa/A hi  [C0][QA_LD]
    static constexpr int B_KL = B_KH + C0 * QA_LD * 2;   // kappa/A lo
    static constexpr int B_WH = B_KL + C0 * QA_LD * 2;   // W^T hi      [M][WT_LD]
    static constexpr int B_WL = B_WH + M * WT_LD * 2;    // W^T lo
    static constexpr int B_AE = B_WL + M * WT_LD * 2;    // A_end       [M] fp32
    static constexpr int B_AR = B_AE + M * 4;            // a_ref       [M] fp32 (see half_product)
    static constexpr int NPT = TB * (TB + 1) / 2;        // causal P^T tiles (tb, jb <= tb)
    static constexpr int B_P = B_AR + M * 4;             // P^T hi, lo  [NPT][2][64 lanes] bf16 x4
    // first linearisation: Q.A.E hi, lo [C0][QA_LD] (coefficients of Z) and A_end E_end [M] fp32
    static constexpr int B_ZH = B_P + NPT * 2 * 64 * 8;
    static constexpr int B_ZL = B_ZH + (LIN1 ? C0 * QA_LD * 2 : 0);
    static constexpr int B_AZ = B_ZL + (LIN1 ? C0 * QA_LD * 2 : 0);
    static constexpr int SET = B_AZ + (LIN1 ? M * 4 : 0);
    static constexpr int BYTES = 2 * SET;
    static_assert(M % 16 == 0 && D % 16 == 0 && C0 % 16 == 0, "tile multiples");
};

template <int M, int D, int C0, bool LIN1 = false>
constexpr bool readout_fits() {
    return ReadCfg<M, D, C0, LIN1>::BYTES <= 160 * 1024;
}

// Register inputs of one sub-block for one lane.
template <class G>
struct RdIn {
    f32x4 g[G::MPW][G::TB], k[G::MPW][G::TB];  // slot 16mb + lc, tokens 16tb + 4lg + (0..3)
    f32x4 e[G::MPW][G::TB];                     // first linearisation only
    f32x4 h[G::TB];                             // column 16w + lc, same tokens
    uint16_t q[G::MPW][G::TB][4];               // q of those (token, slot) pairs, bf16
};

// Waves without a slot tile in the gate phase (more column tiles than slot
// tiles) load only h.
template <class G>
__device__ __forceinline__ void rd_load(RdIn<G>& in, const Params& p, const Workspace& ws, int b, int hd, int t0,
                                        int tc0) {
    constexpr int M = G::MT * 16;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, lc = lane & 15;
    const int C = p.chunk;
    const uint16_t* qg = static_cast<const uint16_t*>(p.q);
#pragma unroll
    for (int mi = 0; mi < G::MPW; ++mi) {
        const int mb = w + mi * G::NW;
        if (mb >= G::MT) continue;  // wave-uniform
        const int slot = 16 * mb + lc;
#pragma unroll
        for (int tb = 0; tb < G::TB; ++tb) {
            const int64_t o = ws_frag(mb, tc0 / 16 + tb, C / 16, lane);
            in.g[mi][tb] = *reinterpret_cast<const f32x4*>(ws.g + o);
            in.k[mi][tb] = *reinterpret_cast<const f32x4*>(ws.k + o);
            if constexpr (G::LIN1_) in.e[mi][tb] = *reinterpret_cast<const f32x4*>(ws.e + o);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int64_t row = (static_cast<int64_t>(b) * p.T + t0 + 16 * tb + 4 * lg + r) * p.H + hd;
                in.q[mi][tb][r] = qg[row * M + slot];
            }
        }
    }
#pragma unroll
    for (int tb = 0; tb < G::TB; ++tb)
        in.h[tb] = *reinterpret_cast<const f32x4*>(ws.h + ws_frag(w, tc0 / 16 + tb, C / 16, lane));
}

// Z of a chunk, stored as its bf16 hi/lo split in this kernel's accumulator
// layout (one 16-byte piece per lane and slot tile).  The pieces stay packed
// in registers until the chunk starts (converting at the load would make the
// load's latency wait there); hi + lo is exact in fp32 and splits back into
// the same hi and lo.
template <int M, int D>
__device__ __forceinline__ void rd_load_z(u32x4 (&z)[M / 16], const float* src) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
    for (int mt = 0; mt < M / 16; ++mt) z[mt] = *reinterpret_cast<const u32x4*>(src + z_frag<D>(mt, w, lane));
}
__device__ __forceinline__ void rd_unpack_z1(f32x4& z, const u32x4& v) {
    z[0] = __uint_as_float(v[0] << 16) + __uint_as_float(v[2] << 16);
    z[1] = __uint_as_float(v[0] & 0xffff0000u) + __uint_as_float(v[2] & 0xffff0000u);
    z[2] = __uint_as_float(v[1] << 16) + __uint_as_float(v[3] << 16);
    z[3] = __uint_as_float(v[1] & 0xffff0000u) + __uint_as_float(v[3] & 0xffff0000u);
}
template <int M>
__device__ __forceinline__ void rd_unpack_z(f32x4 (&z)[M / 16], const u32x4 (&v)[M / 16]) {
#pragma unroll
    for (int mt = 0; mt < M / 16; ++mt) rd_unpack_z1(z[mt], v[mt]);
}

// LIN1: the first chunk linearisation (eq. recurrence_linear1): every token
// also adds e (.) Z, Z the chunk-start state, so with E_t the running sum of
// e_j / A_j inside the sub-block
//   Y  += (Q (.) A (.) E) Z,   R <- ... + diag(A_end E_end) Z.
template <int M, int D, int C0, bool LIN1 = false>
__global__ __launch_bounds__(4 * D) void osr_readout_kernel(Params p, int cpw) {
    using G = ReadCfg<M, D, C0, LIN1>;
    constexpr int MT = G::MT, TB = G::TB;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    const int C = p.chunk, SPC = C / C0;
    const int n0 = p.n_begin, n1 = p.n_end > 0 ? p.n_end : p.T / C;  // chunk range of this launch
    const int groups = (n1 - n0) / cpw;
    const int bh = blockIdx.x / groups, grp = blockIdx.x % groups;
    const int b = bh / p.H, hd = bh % p.H;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, lc = lane & 15;
    const int dcol = 16 * w + lc;
    const int ch0 = n0 + grp * cpw, NS = cpw * SPC;
    const s16x4 eye = eye_operand(false);

    f32x4 acc[MT];  // R tiles: acc[mt][r] = R[16mt + 4lg + r][dcol]
    u32x4 zn[MT];   // next chunk's Z (packed hi/lo)
    u32x4 zc[MT];   // this chunk's Z (packed hi/lo; first linearisation)
    RdIn<G> cur, nxt;
    {
        const Workspace ws = workspace_at<M, D>(p, bh, ch0);
        rd_load_z<M, D>(zn, ws.z);
        rd_unpack_z<M>(acc, zn);
        if constexpr (LIN1) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) zc[mt] = zn[mt];
        }
        rd_load<G>(cur, p, ws, b, hd, ch0 * C, 0);
    }
    for (int s = 0; s < NS; ++s) {
        const int sl = s % SPC, n = ch0 + s / SPC;
        const int tc0 = sl * C0, t0 = n * C + tc0;
        char* buf = smem + (s & 1) * G::SET;
        short* qah = reinterpret_cast<short*>(buf + G::B_QH);
        short* qal = reinterpret_cast<short*>(buf + G::B_QL);
        short* kah = reinterpret_cast<short*>(buf + G::B_KH);
        short* kal = reinterpret_cast<short*>(buf + G::B_KL);
        short* wth = reinterpret_cast<short*>(buf + G::B_WH);
        short* wtl = reinterpret_cast<short*>(buf + G::B_WL);
        float* aend = reinterpret_cast<float*>(buf + G::B_AE);
        float* arefs = reinterpret_cast<float*>(buf + G::B_AR);
        short* zqh = reinterpret_cast<short*>(buf + G::B_ZH);
        short* zql = reinterpret_cast<short*>(buf + G::B_ZL);
        float* aez = reinterpret_cast<float*>(buf + G::B_AZ);
        const bool last_in_chunk = sl + 1 == SPC;

        // Inputs of the next sub-block (the last one re-reads its own).
        {
            const int s1 = s + 1 < NS ? s + 1 : s;
            const int n1 = ch0 + s1 / SPC, tc1 = (s1 % SPC) * C0;
            const Workspace ws1 = workspace_at<M, D>(p, bh, n1);
            rd_load<G>(nxt, p, ws1, b, hd, n1 * C + tc1, tc1);
            if (last_in_chunk) rd_load_z<M, D>(zn, ws1.z);
        }

        // The post-gate of this sub-block's y (if fused), loaded here so the
        // loads land while the products below run: lane (lg, lc) reads 4
        // consecutive columns of token row lc (8 bytes; 16 lanes cover a 32-byte
        // row piece), and the identity product brings them into the layout of y.
        s16x4 gq[TB] = {};
        if (p.gate) {
            const short* gp = static_cast<const short*>(p.gate);
            const int64_t g0 = (static_cast<int64_t>(b) * p.T + t0) * p.H + hd;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
                gq[tb] = *reinterpret_cast<const s16x4*>(gp + (g0 + static_cast<int64_t>(16 * tb + lc) * p.H) * D + 16 * w + 4 * lg);
        }

        // ---- gate products of this wave's slot tiles ------------------------
#pragma unroll
        for (int mi = 0; mi < G::MPW; ++mi) {
            const int mb = w + mi * G::NW;
            if (mb < MT) {
                const int slot = 16 * mb + lc;
                float below[TB], above[TB], tot[TB], first_rows = 1.f;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const f32x4 g = cur.g[mi][tb];
                    const float x = g[0] * g[1] * g[2] * g[3];
                    rows4_prod_scan(x, lg, below[tb], above[tb], tot[tb]);
                    if (TB == 1) first_rows = rows01_prod(x);
                }
                // A (running product, inclusive, relative to a_ref), Q.A and
                // kappa/A, token-major; first linearisation: E (running sum of
                // e/A, inclusive) and Q.A.E.
                const float aref = half_product<TB>(tot, first_rows);
                float fwd = 1.f / aref, esum = 0.f;
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const f32x4 g = cur.g[mi][tb], kp = cur.k[mi][tb];
                    float a = fwd * below[tb];
                    float E = 0.f;
                    f32x4 ea;
                    if constexpr (LIN1) {
                        // e/A of this lane's tokens, then the sums of the lane rows below
                        const f32x4 e = cur.e[mi][tb];
                        float a2 = a, es = 0.f;
#pragma unroll
                        for (int r = 0; r < 4; ++r) {
                            a2 *= g[r];
                            ea[r] = e[r] / a2;
                            es += ea[r];
                        }
                        float es_below, es_tot;
                        rows4_sum_scan(es, lg, es_below, es_tot);
                        E = esum + es_below;
                        esum += es_tot;
                    }
                    f32x4 qa, ka, qz;
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        a *= g[r];
                        qa[r] = bf16u(cur.q[mi][tb][r]) * a;
                        ka[r] = kp[r] / a;
                        if constexpr (LIN1) {
                            E += ea[r];
                            qz[r] = qa[r] * E;
                        }
                    }
                    s16x4 qh, ql, kh, kl;
                    split4(qa, qh, ql);
                    split4(ka, kh, kl);
                    // transposed, the lane holds slots 16mb + 4lg .. +3 of token 16tb + lc
                    const int o = (16 * tb + lc) * G::QA_LD + 16 * mb + 4 * lg;
                    *reinterpret_cast<s16x4*>(qah + o) = tr16(qh, eye);
                    *reinterpret_cast<s16x4*>(qal + o) = tr16(ql, eye);
                    *reinterpret_cast<s16x4*>(kah + o) = tr16(kh, eye);
                    *reinterpret_cast<s16x4*>(kal + o) = tr16(kl, eye);
                    if constexpr (LIN1) {
                        s16x4 zh, zl;
                        split4(qz, zh, zl);
                        *reinterpret_cast<s16x4*>(zqh + o) = tr16(zh, eye);
                        *reinterpret_cast<s16x4*>(zql + o) = tr16(zl, eye);
                    }
                    fwd *= tot[tb];
                }
                // W_t = kappa_t (.) prod_{l > t} g_l, slot-major.
                float bwd = 1.f;
#pragma unroll
                for (int tb = TB - 1; tb >= 0; --tb) {
                    const f32x4 g = cur.g[mi][tb], kp = cur.k[mi][tb];
                    float sfx = bwd * above[tb];
                    f32x4 wv;
#pragma unroll
                    for (int r = 3; r >= 0; --r) {
                        wv[r] = kp[r] * sfx;
                        sfx *= g[r];
                    }
                    s16x4 wh, wl;
                    split4(wv, wh, wl);
                    *reinterpret_cast<s16x4*>(wth + slot * G::WT_LD + 16 * tb + 4 * lg) = wh;
                    *reinterpret_cast<s16x4*>(wtl + slot * G::WT_LD + 16 * tb + 4 * lg) = wl;
                    bwd *= tot[tb];
                }
                if (lg == 0) {
                    aend[slot] = fwd * aref;
                    arefs[slot] = aref;
                    if constexpr (LIN1) aez[slot] = fwd * esum;  // A_end E_end: the a_ref factors cancel
                }
            }
        }
        __syncthreads();  // Q.A, kappa/A, W^T, A_end visible

        // ---- Y = (Q.A) R + tril(P) H, P^T = (kappa/A)(Q.A)^T ------------------
        // R scaled by a_ref per slot (the Q.A tiles are relative to it)
        s16x4 rh[MT], rl[MT], hh[TB], hl[TB];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 ar = *reinterpret_cast<const f32x4*>(arefs + 16 * mt + 4 * lg);
            f32x4 rs = acc[mt];
#pragma unroll
            for (int r = 0; r < 4; ++r) rs[r] *= ar[r];
            split4(rs, rh[mt], rl[mt]);
        }
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) split4(cur.h[tb], hh[tb], hl[tb]);
        const int64_t row0 = (static_cast<int64_t>(b) * p.T + t0) * p.H + hd;
        // The causal tiles P^T (tb, jb <= tb) do not depend on the wave's
        // columns: tile k = tb(tb+1)/2 + jb is formed once, by wave k % NW
        // (masked, split), and shared through LDS in lane order; meanwhile
        // every wave forms (Q.A) R for its columns.
        // 16x16x16 products here: the same contractions as 16x16x32 on
        // permuted operands gave wrong results on gfx950 in this kernel
        // (correct once nops padded the MFMA sequence), so this path keeps
        // the 16-deep form, which is exact to rounding.
        short* pbuf = reinterpret_cast<short*>(buf + G::B_P);
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int jb = 0; jb <= tb; ++jb) {
                const int k = tb * (tb + 1) / 2 + jb;
                if (k % G::NW == w) {
                    f32x4 pj = {0.f, 0.f, 0.f, 0.f};  // lane (lg, lc): P^T[16jb + 4lg + r][16tb + lc]
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt) {
                        const int qo = (16 * tb + lc) * G::QA_LD + 16 * mt + 4 * lg;
                        const int ko = (16 * jb + lc) * G::QA_LD + 16 * mt + 4 * lg;
                        pj = mma3(ld4s(kah + ko), ld4s(kal + ko), ld4s(qah + qo), ld4s(qal + qo), pj);
                    }
                    if (jb == tb) {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (4 * lg + r > lc) pj[r] = 0.f;  // causal: j <= t
                    }
                    s16x4 ph, pl;
                    split4(pj, ph, pl);
                    *reinterpret_cast<s16x4*>(pbuf + ((2 * k) * 64 + lane) * 4) = ph;
                    *reinterpret_cast<s16x4*>(pbuf + ((2 * k + 1) * 64 + lane) * 4) = pl;
                }
            }
        f32x4 yt[TB];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            yt[tb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const int qo = (16 * tb + lc) * G::QA_LD + 16 * mt + 4 * lg;
                yt[tb] = mma3(ld4s(qah + qo), ld4s(qal + qo), rh[mt], rl[mt], yt[tb]);
                if constexpr (LIN1) {
                    // (Q.A.E) Z with Z's own hi/lo split as the B operand
                    const s16x4 zh = __builtin_bit_cast(s16x4, u32x2{zc[mt][0], zc[mt][1]});
                    const s16x4 zl = __builtin_bit_cast(s16x4, u32x2{zc[mt][2], zc[mt][3]});
                    yt[tb] = mma3(ld4s(zqh + qo), ld4s(zql + qo), zh, zl, yt[tb]);
                }
            }
        }
        __syncthreads();  // P^T tiles visible
#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            f32x4 y = yt[tb];
#pragma unroll
            for (int jb = 0; jb <= tb; ++jb) {
                const int k = tb * (tb + 1) / 2 + jb;
                const s16x4 ph = *reinterpret_cast<const s16x4*>(pbuf + ((2 * k) * 64 + lane) * 4);
                const s16x4 pl = *reinterpret_cast<const s16x4*>(pbuf + ((2 * k + 1) * 64 + lane) * 4);
                y = mma3(ph, pl, hh[jb], hl[jb], y);
            }
            // 4-byte stores: 16 lanes cover 64 contiguous bytes of a token row
            // (a transposed tile, 16 bytes per lane across 16 rows, issues four
            // times the memory requests)
            if (p.gate) {
                const f32x4 gf = tr16f(gq[tb], eye);  // gate of tokens 16tb + 4lg + r, column dcol
#pragma unroll
                for (int r = 0; r < 4; ++r) y[r] *= gelu(gf[r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                st_y1(p.y, (row0 + static_cast<int64_t>(16 * tb + 4 * lg + r) * p.H) * D + dcol, y[r], p.y_bf16);
        }

        // ---- R <- diag(A_end) R + W^T H (next sub-block of the same chunk) ----
        if (!last_in_chunk) {
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const f32x4 ae = *reinterpret_cast<const f32x4*>(aend + 16 * mt + 4 * lg);
                f32x4 a = acc[mt];
#pragma unroll
                for (int r = 0; r < 4; ++r) a[r] *= ae[r];
                if constexpr (LIN1) {
                    const f32x4 az = *reinterpret_cast<const f32x4*>(aez + 16 * mt + 4 * lg);
                    f32x4 zf;
                    rd_unpack_z1(zf, zc[mt]);
#pragma unroll
                    for (int r = 0; r < 4; ++r) a[r] = fmaf(zf[r], az[r], a[r]);
                }
                if constexpr (G::K32_C) {
#pragma unroll
                    for (int kt = 0; kt < C0 / 32; ++kt) {
                        const int wo = (16 * mt + lc) * G::WT_LD + 32 * kt + 4 * lg;
                        a = mma32x3(ld8p(wth + wo), ld8p(wtl + wo), cat8(hh[2 * kt], hh[2 * kt + 1]),
                                    cat8(hl[2 * kt], hl[2 * kt + 1]), a);
                    }
                } else {
                    const int wo = (16 * mt + lc) * G::WT_LD + 4 * lg;
                    a = mma3(ld4s(wth + wo), ld4s(wtl + wo), hh[0], hl[0], a);
                }
                acc[mt] = a;
            }
        } else {
            rd_unpack_z<M>(acc, zn);
            if constexpr (LIN1) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) zc[mt] = zn[mt];
            }
        }
        cur = nxt;
    }
}

}  // namespace mfma
}  // namespace osr
