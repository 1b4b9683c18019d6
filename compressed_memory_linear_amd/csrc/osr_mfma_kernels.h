// osr_mfma_kernels.h -- chunk-wise OSR forward on gfx950 matrix cores: shared
// operand helpers, input staging, the workspace layout and the fused kernel
// (the split schedule's kernels are in osr_mfma_chain.h and osr_mfma_readout.h).
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
// over sub-blocks of C0 tokens: with A the running product of g inside the
// sub-block and R the running state at its start,
//   Y   = (Q (.) A) R + tril[(Q (.) A)(kappa (/) A)^T] H
//   R  <- diag(A_end) R + W^T H,   W_t = kappa_t (.) prod_{l > t} g_l.
// Z and R are fp32; every product whose operand derives from the state runs
// as three bf16 MFMAs on a hi/lo split (hi*hi + hi*lo + lo*hi); k and q are
// exact bf16 inputs.
//
// Fused kernel's work layout: one workgroup of D/16 waves; wave w owns columns
// [16w, 16w + 16) of the state (as MFMA accumulators), of H and of Y.  With
// v_mfma_f32_16x16x16_bf16 an accumulator tile (lane l holds rows
// 4(l/16)+r of column l%16) is directly a B operand whose k index is the
// tile's row, so R feeds the read-out and H feeds the causal product and the
// state update without a transpose.  The contraction over d (c = H Z^T) goes
// through LDS; the wave that owns slot block mb computes c for all tokens of
// the sub-block and forms the gates and their running/suffix products in
// registers (lane shuffles), so a sub-block needs two workgroup barriers.
// Inputs of sub-block s+1 are loaded into registers while s computes.
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

// v_mfma_f32_16x16x32_bf16: twice the k of the 16x16x16 form at the same
// issue cost.  Lane l holds A[l%16][8(l/16)+j] and B[8(l/16)+j][l%16].
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x4 mma32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32x3(bf16x8 ah, bf16x8 al, bf16x8 bh, bf16x8 bl, f32x4 c) {
    c = mma32(al, bh, c);
    c = mma32(ah, bl, c);
    return mma32(ah, bh, c);
}
__device__ __forceinline__ bf16x8 ld8(const short* p) { return *reinterpret_cast<const bf16x8*>(p); }

__device__ __forceinline__ short bf16_bits(float x) {
    return __builtin_bit_cast(short, static_cast<__bf16>(x));
}
__device__ __forceinline__ float bf16_val(short b) {
    return __uint_as_float(static_cast<uint32_t>(static_cast<uint16_t>(b)) << 16);
}
__device__ __forceinline__ float bf16u(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// x = hi + lo with hi = bf16(x), lo = bf16(x - hi) (round to nearest even).
__device__ __forceinline__ void split1(float x, short& hi, short& lo) {
    hi = bf16_bits(x);
    lo = bf16_bits(x - bf16_val(hi));
}
// Four values at a time: packed conversions of pairs; the hi part of each
// pair comes back as fp32 with a shift (low half) or a mask (high half).
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned cvt2_bf16(float a, float b) {
    return __builtin_bit_cast(unsigned, __builtin_convertvector(f32x2{a, b}, bf16x2));
}
__device__ __forceinline__ void split4(f32x4 x, s16x4& hi, s16x4& lo) {
    const unsigned h01 = cvt2_bf16(x[0], x[1]), h23 = cvt2_bf16(x[2], x[3]);
    const float r0 = x[0] - __uint_as_float(h01 << 16), r1 = x[1] - __uint_as_float(h01 & 0xffff0000u);
    const float r2 = x[2] - __uint_as_float(h23 << 16), r3 = x[3] - __uint_as_float(h23 & 0xffff0000u);
    hi = __builtin_bit_cast(s16x4, u32x2{h01, h23});
    lo = __builtin_bit_cast(s16x4, u32x2{cvt2_bf16(r0, r1), cvt2_bf16(r2, r3)});
}

// 16x16x32 operands built from accumulator tiles use a permuted k order: two
// D-layout tiles t0, t1 (lane (lg, lc) holds rows 4lg..4lg+3 of column lc)
// concatenated form an operand whose k index 8lg + j stands for row
// 16(j/4) + 4lg + j%4 of the 32-row block; the matching operand is read from
// LDS as two 8-byte pieces at columns 4lg and 16 + 4lg of the block.  Any
// bijection of k leaves the contraction unchanged.
typedef short s16x8 __attribute__((ext_vector_type(8)));

// Two D-layout tiles -> one permuted 32-k operand.
__device__ __forceinline__ bf16x8 cat8(s16x4 a, s16x4 b) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}
// The matching operand read from LDS: p points at column 4lg of a 32-column block.
__device__ __forceinline__ bf16x8 ld8p(const short* p) {
    return cat8(*reinterpret_cast<const s16x4*>(p), *reinterpret_cast<const s16x4*>(p + 16));
}
__device__ __forceinline__ s16x4 ld4s(const short* p) { return *reinterpret_cast<const s16x4*>(p); }

// Tile transposes on the matrix core.  A lane passes the four values it holds
// in the accumulator layout, X[4lg + r][lc], as an A operand, which reads them
// as A[lc][4lg + r], i.e. X^T; times the identity the product returns in the
// accumulator layout, so the lane then holds X[lc][4lg + r]: four consecutive
// columns of row lc, one 8-byte LDS access instead of four 2-byte ones.  The
// same product turns four consecutive bf16 values of row lc read from LDS
// into the accumulator layout (fp32).  Every product is x * 1 or x * 0, so the
// results are the bf16 inputs exactly (times -1 with the negated identity).
__device__ __forceinline__ s16x4 eye_operand(bool negate) {
    const int lane = threadIdx.x & 63, lg = lane >> 4, lc = lane & 15;
    const short one = negate ? static_cast<short>(0xBF80) : static_cast<short>(0x3F80);
    s16x4 e;
#pragma unroll
    for (int j = 0; j < 4; ++j) e[j] = 4 * lg + j == lc ? one : static_cast<short>(0);
    return e;
}
__device__ __forceinline__ f32x4 tr16f(s16x4 x, s16x4 eye) { return mma(x, eye, f32x4{0.f, 0.f, 0.f, 0.f}); }
__device__ __forceinline__ s16x4 tr16(s16x4 x, s16x4 eye) {
    const f32x4 t = tr16f(x, eye);  // bf16 values: the conversions are exact
    return __builtin_bit_cast(s16x4, u32x2{cvt2_bf16(t[0], t[1]), cvt2_bf16(t[2], t[3])});
}

// Reductions over the four 16-lane rows of a wave, per lane column, with the
// gfx950 row swaps: permlane16_swap(x, x) gives every row the value of the
// even and of the odd row of its pair (rows 0/1, 2/3); permlane32_swap(y, y)
// gives the values of rows 0/1 and of rows 2/3 when y is uniform per pair.
__device__ __forceinline__ void pair_rows(float x, float& even, float& odd) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    even = __uint_as_float(r[0]);
    odd = __uint_as_float(r[1]);
}
__device__ __forceinline__ void half_rows(float y, float& lo, float& hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}
__device__ __forceinline__ float rows4_sum(float x) {
    float e, o, lo, hi;
    pair_rows(x, e, o);
    half_rows(e + o, lo, hi);
    return lo + hi;
}
// Sums over the rows of x per lane column: below = rows < lg, total = all four.
__device__ __forceinline__ void rows4_sum_scan(float x, int lg, float& below, float& total) {
    float e, o, lo, hi;
    pair_rows(x, e, o);
    half_rows(e + o, lo, hi);
    total = lo + hi;
    below = ((lg & 1) ? e : 0.f) + ((lg & 2) ? lo : 0.f);
}
// Products over the rows of x per lane column: below = rows < lg, above =
// rows > lg, total = all four.
__device__ __forceinline__ void rows4_prod_scan(float x, int lg, float& below, float& above, float& total) {
    float e, o, lo, hi;
    pair_rows(x, e, o);
    half_rows(e * o, lo, hi);
    total = lo * hi;
    below = ((lg & 1) ? e : 1.f) * ((lg & 2) ? lo : 1.f);
    above = ((lg & 1) ? 1.f : o) * ((lg & 2) ? 1.f : hi);
}

// Product of the first two of the four 16-lane rows of x, per lane column
// (the first 8 tokens of a 16-token tile when each row holds 4 of them).
__device__ __forceinline__ float rows01_prod(float x) {
    float e, o, lo, hi;
    pair_rows(x, e, o);
    half_rows(e * o, lo, hi);
    return lo;
}

// Scale reference of the in-sub-block gate products.  The causal part of the
// read-out pairs q_t A_t with kappa_j / A_j, A the running product of g from
// the sub-block start; with small gates A_j underflows (and 1/A_j overflows)
// although every ratio A_t / A_j (j <= t) is a product of gates.  Both factors
// are therefore taken relative to A at the middle of the sub-block, a_ref (the
// product of g over its first half): q_t A_t / a_ref and kappa_j a_ref / A_j,
// whose exponents span half the range each; the (Q.A) R term then takes R
// scaled by a_ref.
template <int TB>
__device__ __forceinline__ float half_product(const float (&tot)[TB], float first_rows) {
    if constexpr (TB == 1) {
        return first_rows;
    } else {
        float a = 1.f;
#pragma unroll
        for (int tb = 0; tb < TB / 2; ++tb) a *= tot[tb];
        return a;
    }
}

// Workspace of the split schedule, fp32, for every (b,h) and chunk n (all
// taken at the chunk-start state): Z [m][d], the gates g and kappa and the
// vectors h (and, with the first linearisation, the coefficient e of the
// chunk-start slot in each token's update).  The state-passing kernel writes it, the read-out kernel reads it.
// g, kappa (per slot block) and h (per column block) are stored in MFMA lane
// order, 1 KiB per (16-row block, 16-token tile): lane (lg, lc) holds row
// 16*block + lc at tokens 16*tile + 4*lg .. +3.  Both kernels hold them in
// exactly that lane layout, so every store and load moves one contiguous KiB.
struct Workspace {
    float* z;
    float* g;
    float* k;
    float* h;
    float* e;  // first linearisation only: the chunk-start term's coefficient beta a c
};
// Offset (floats) of the 4 values of one lane: block of 16 rows, token tile
// of the chunk (C/16 tiles per block).
__device__ __forceinline__ int64_t ws_frag(int block, int tile, int tiles_per_chunk, int lane) {
    return ((static_cast<int64_t>(block) * tiles_per_chunk + tile) * 64 + lane) * 4;
}
// Offset (floats) of one lane's piece of Z: slot block mt, column tile j; the
// piece holds the bf16 hi parts of Z[16mt + 4lg + r][16j + lc], r = 0..3,
// then the lo parts (16 bytes).
template <int D>
__device__ __forceinline__ int64_t z_frag(int mt, int j, int lane) {
    return ((static_cast<int64_t>(mt) * (D / 16) + j) * 64 + lane) * 4;
}
template <int M, int D>
__device__ __forceinline__ Workspace workspace_at(const Params& p, int bh, int n) {
    const int C = p.chunk, NC = p.T / C;
    const int64_t nch = static_cast<int64_t>(p.B) * p.H * NC, i = static_cast<int64_t>(bh) * NC + n;
    float* g0 = p.zbuf + nch * M * D;
    float* k0 = g0 + nch * M * C;
    float* h0 = k0 + nch * M * C;
    float* e0 = h0 + nch * D * C;  // present with the first linearisation only
    return Workspace{p.zbuf + i * M * D, g0 + i * M * C, k0 + i * M * C, h0 + i * D * C,
                     p.lin1 ? e0 + i * M * C : nullptr};
}

template <int M, int D, int C0, bool WITH_Y>
struct Cfg {
    static constexpr int M_ = M, D_ = D, C0_ = C0;
    static constexpr int NW = D / 16;   // waves; wave w owns d-block w
    static constexpr int NT = 64 * NW;
    static constexpr int MT = M / 16;   // slot tiles
    static constexpr int TB = C0 / 16;  // token tiles per sub-block
    static constexpr int MPW = (MT + NW - 1) / NW;  // slot tiles per wave in the gate phase
    static constexpr int PAD = 8;       // bf16 elements of row padding
    static constexpr int ZS_LD = D + PAD;
    static constexpr int KS_LD = M + PAD;
    static constexpr int HS_LD = D + PAD;
    static constexpr int QA_LD = M + PAD;
    static constexpr int WT_LD = C0 + PAD;
    static constexpr int HT_LD = C0 + PAD;
    static constexpr int VS_LD = D + PAD;
    // Which contractions run as 16x16x32 (their k extent is a multiple of 32).
    static constexpr bool K32_M = M % 32 == 0;   // H = K Z (k = slot)
    static constexpr bool K32_D = D % 32 == 0;   // c = H Z^T (k = column)
    static constexpr bool K32_C = C0 % 32 == 0;  // R += W^T H (k = token)
    static constexpr int GS_LD = M;                        // gamma / q tiles (unpadded)
    // 16-byte pieces of the staged tiles, and pieces per thread.
    static constexpr int KPC = C0 * M / 8, KPT = (KPC + NT - 1) / NT;
    static constexpr int VPC = C0 * D / 8, VPT = (VPC + NT - 1) / NT;
    // One staging buffer: K [C0][KS_LD], V [C0][VS_LD], gamma [C0][M] (a
    // per-token gamma broadcast over the slots), q [C0][M] (read-out only) in
    // bf16; mu [C0] in fp32.
    static constexpr int SO_K = 0;
    static constexpr int SO_V = SO_K + C0 * KS_LD;
    static constexpr int SO_G = SO_V + C0 * VS_LD;
    static constexpr int SO_Q = SO_G + C0 * GS_LD;
    static constexpr int SO_MU = SO_Q + (WITH_Y ? C0 * GS_LD : 0);  // mu [C0] fp32
    static constexpr int STAGE = SO_MU + 2 * C0;           // bf16 elements per buffer

    // LDS layout (bytes).
    static constexpr int O_ZH = 0;                                  // Z hi  [M][ZS_LD]
    static constexpr int O_ZL = O_ZH + M * ZS_LD * 2;               // Z lo
    static constexpr int O_KS = O_ZL + M * ZS_LD * 2;               // staging [2][STAGE]
    static constexpr int O_HH = O_KS + 2 * STAGE * 2;               // H hi  [C0][HS_LD]
    static constexpr int O_HL = O_HH + C0 * HS_LD * 2;              // H lo
    static constexpr int O_HP = O_HL + C0 * HS_LD * 2;              // |h|^2 partials [NW][C0]
    static constexpr int O_TH = O_HP + NW * C0 * 4;                 // H^T hi [D][HT_LD]
    static constexpr int O_TL = O_TH + (K32_C ? D * HT_LD * 2 : 0); // H^T lo
    static constexpr int O_WH = O_TL + (K32_C ? D * HT_LD * 2 : 0); // W^T hi [M][WT_LD]
    static constexpr int O_WL = O_WH + M * WT_LD * 2;               // W^T lo
    static constexpr int O_AE = O_WL + M * WT_LD * 2;               // A_end [M]
    static constexpr int O_AR = O_AE + M * 4;                       // a_ref [M] (see half_product)
    static constexpr int O_NP = O_AR + M * 4;                       // norm partials [NW][M]
    static constexpr int O_QH = O_NP + NW * M * 4;                  // Q.A hi [C0][QA_LD]
    static constexpr int O_QL = O_QH + (WITH_Y ? C0 * QA_LD * 2 : 0);
    static constexpr int O_KH = O_QL + (WITH_Y ? C0 * QA_LD * 2 : 0);  // kappa/A hi
    static constexpr int O_KL = O_KH + (WITH_Y ? C0 * QA_LD * 2 : 0);
    static constexpr int BYTES = O_KL + (WITH_Y ? C0 * QA_LD * 2 : 0);

    static_assert(M % 16 == 0 && D % 16 == 0 && C0 % 16 == 0, "tile multiples");
    static_assert(NW >= 1 && NT <= 1024, "waves");
};

template <int M, int D, int C0, bool WITH_Y>
constexpr bool fits() {
    return Cfg<M, D, C0, WITH_Y>::BYTES <= 160 * 1024;
}

// Inputs of the next sub-block, loaded into registers as 16-byte pieces while
// the current sub-block computes and written to its LDS staging buffer only
// after the current sub-block's gate phase (so the loads have a whole phase
// of work to land behind).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <class G>
struct Pre {
    u32x4 k[G::KPT], g[G::KPT], q[G::KPT], v[G::VPT];
    uint16_t gtok[G::KPT];  // per-token gamma of each piece's token
    uint16_t mu;            // thread tau < C0 holds token tau
};

// Per-lane byte offsets of a thread's staged pieces, relative to the
// sub-block's first token row of its (b, h).  They do not change from one
// sub-block to the next (only the wave-uniform base does), so they are
// computed once and every load is a uniform 64-bit base plus a 32-bit lane
// offset.
template <class G>
struct PreOff {
    uint32_t kq[G::KPT];   // k, a per-slot gamma tile and q pieces
    uint32_t gtok[G::KPT]; // gamma of each k piece's token (per-token gamma), or its first slot
    uint32_t v[G::VPT];
    uint32_t mu;
};

template <class G>
__device__ __forceinline__ PreOff<G> prefetch_offsets(const Params& p) {
    constexpr int M = G::M_, D = G::D_, C0 = G::C0_;
    const int tid = threadIdx.x;
    const uint32_t rs = static_cast<uint32_t>(p.H);  // token stride in rows
    PreOff<G> o;
#pragma unroll
    for (int j = 0; j < G::KPT; ++j) {
        int e = tid + j * G::NT;
        if (G::KPC % G::NT != 0) e = e < G::KPC ? e : G::KPC - 1;
        const uint32_t row = static_cast<uint32_t>(e / (M / 8)) * rs;
        o.kq[j] = (row * M + (e % (M / 8)) * 8) * 2;
        o.gtok[j] = (p.gamma_per_slot ? row * M : row) * 2;
    }
#pragma unroll
    for (int j = 0; j < G::VPT; ++j) {
        int e = tid + j * G::NT;
        if (G::VPC % G::NT != 0) e = e < G::VPC ? e : G::VPC - 1;
        o.v[j] = (static_cast<uint32_t>(e / (D / 8)) * rs * D + (e % (D / 8)) * 8) * 2;
    }
    o.mu = static_cast<uint32_t>(tid % C0) * rs * 2;
    return o;
}

// Every load below is unconditional (indices are clamped) so none sits behind
// a branch, which would make the compiler wait for it at the join.  A
// per-token gamma is broadcast over the 8 slots of each piece at commit, so the
// staged gamma tile is always [C0][M]: both the tile load (a valid dummy tile,
// k, for a per-token gamma) and the scalar load (the first slot's gamma for a
// per-slot gamma) are issued, and commit picks one.
template <class G, bool WITH_Y>
__device__ __forceinline__ void prefetch(Pre<G>& pf, const PreOff<G>& o, const Params& p, int b, int hd, int t0) {
    constexpr int M = G::M_, D = G::D_;
    const bool gslot = p.gamma_per_slot != 0;
    const int64_t row0 = (static_cast<int64_t>(b) * p.T + t0) * p.H + hd;  // token t0
    const char* kb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.k) + row0 * M);
    const char* gb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.gamma) + (gslot ? row0 * M : row0));
    const char* tb = gslot ? gb : kb;  // per-slot gamma tile, or a valid dummy
    const char* qb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.q) + row0 * M);
    const char* vb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.v) + row0 * D);
    const char* mb = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.mu) + row0);
#pragma unroll
    for (int j = 0; j < G::KPT; ++j) {
        pf.k[j] = *reinterpret_cast<const u32x4*>(kb + o.kq[j]);
        pf.g[j] = *reinterpret_cast<const u32x4*>(tb + o.kq[j]);
        pf.gtok[j] = *reinterpret_cast<const uint16_t*>(gb + o.gtok[j]);
        if constexpr (WITH_Y) pf.q[j] = *reinterpret_cast<const u32x4*>(qb + o.kq[j]);
    }
#pragma unroll
    for (int j = 0; j < G::VPT; ++j) pf.v[j] = *reinterpret_cast<const u32x4*>(vb + o.v[j]);
    pf.mu = *reinterpret_cast<const uint16_t*>(mb + o.mu);
}

template <class G, bool WITH_Y>
__device__ __forceinline__ void commit(const Pre<G>& pf, short* st, bool gslot) {
    constexpr int M = G::M_, D = G::D_, C0 = G::C0_;
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < G::KPT; ++j) {
        const int e = tid + j * G::NT;
        if (G::KPC % G::NT == 0 || e < G::KPC) {
            const int tau = e / (M / 8), i0 = (e % (M / 8)) * 8;
            *reinterpret_cast<u32x4*>(st + G::SO_K + tau * G::KS_LD + i0) = pf.k[j];
            const unsigned g2 = static_cast<unsigned>(pf.gtok[j]) * 0x10001u;
            *reinterpret_cast<u32x4*>(st + G::SO_G + tau * G::GS_LD + i0) = gslot ? pf.g[j] : u32x4{g2, g2, g2, g2};
            if constexpr (WITH_Y) *reinterpret_cast<u32x4*>(st + G::SO_Q + tau * G::GS_LD + i0) = pf.q[j];
        }
    }
#pragma unroll
    for (int j = 0; j < G::VPT; ++j) {
        const int e = tid + j * G::NT;
        if (G::VPC % G::NT == 0 || e < G::VPC) {
            const int tau = e / (D / 8), c0 = (e % (D / 8)) * 8;
            *reinterpret_cast<u32x4*>(st + G::SO_V + tau * G::VS_LD + c0) = pf.v[j];
        }
    }
    if (tid < C0) reinterpret_cast<float*>(st + G::SO_MU)[tid] = bf16u(pf.mu);
}

// Products of x over the four 16-lane groups of a wave, per lane column:
// excl_lo = prod over lower groups, excl_hi = prod over higher groups,
// total = prod over all four.
__device__ __forceinline__ void group_scan(float x, int lg, float& excl_lo, float& excl_hi, float& total) {
    float inc = x;
    float t = __shfl_up(inc, 16, 64);
    if (lg >= 1) inc *= t;
    t = __shfl_up(inc, 32, 64);
    if (lg >= 2) inc *= t;
    // inc = prod_{g' <= lg}
    t = __shfl_up(inc, 16, 64);
    excl_lo = lg >= 1 ? t : 1.f;
    const int lane = threadIdx.x & 63;
    total = __shfl(inc, (lane & 15) + 48, 64);
    float sinc = x;
    t = __shfl_down(sinc, 16, 64);
    if (lg <= 2) sinc *= t;
    t = __shfl_down(sinc, 32, 64);
    if (lg <= 1) sinc *= t;
    // sinc = prod_{g' >= lg}
    t = __shfl_down(sinc, 16, 64);
    excl_hi = lg <= 2 ? t : 1.f;
}

// --------------------------------------------------------------------------
// One sub-block of C0 tokens starting at token t0 (inside a chunk whose
// chunk-start state Z is in zfh/zfl and in LDS).  acc_R: running state.
// st: this sub-block's staged inputs (visible); nxt: the next sub-block's
// inputs (in flight), written to st_next here.
template <int M, int D, int C0, bool WITH_Y>
__device__ __forceinline__ void osr_subblock(const Params& p, char* smem, f32x4 (&acc_R)[M / 16],
                                             const s16x4 (&zfh)[M / 16], const s16x4 (&zfl)[M / 16],
                                             const bf16x8 (&z8h)[(M + 31) / 32], const bf16x8 (&z8l)[(M + 31) / 32],
                                             bool r_is_z, const short* st,
                                             const Pre<Cfg<M, D, C0, WITH_Y>>& nxt, short* st_next,
                                             bool has_next, bool need_state, int b, int hd, int t0) {
    using G = Cfg<M, D, C0, WITH_Y>;
    constexpr int MT = G::MT, TB = G::TB;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lg = lane >> 4, lc = lane & 15;
    const int dcol = 16 * w + lc;
    const short* ks = st + G::SO_K;
    const short* vs = st + G::SO_V;
    const short* gs = st + G::SO_G;
    const short* qs = st + G::SO_Q;
    const float* mus = reinterpret_cast<const float*>(st + G::SO_MU);

    short* zh = reinterpret_cast<short*>(smem + G::O_ZH);
    short* zl = reinterpret_cast<short*>(smem + G::O_ZL);
    short* hsh = reinterpret_cast<short*>(smem + G::O_HH);
    short* hsl = reinterpret_cast<short*>(smem + G::O_HL);
    float* hp = reinterpret_cast<float*>(smem + G::O_HP);
    short* hth = reinterpret_cast<short*>(smem + G::O_TH);
    short* htl = reinterpret_cast<short*>(smem + G::O_TL);
    short* wth = reinterpret_cast<short*>(smem + G::O_WH);
    short* wtl = reinterpret_cast<short*>(smem + G::O_WL);
    float* aend = reinterpret_cast<float*>(smem + G::O_AE);
    float* arefs = reinterpret_cast<float*>(smem + G::O_AR);
    short* qah = reinterpret_cast<short*>(smem + G::O_QH);
    short* qal = reinterpret_cast<short*>(smem + G::O_QL);
    short* kah = reinterpret_cast<short*>(smem + G::O_KH);
    short* kal = reinterpret_cast<short*>(smem + G::O_KL);

    // The post-gate of this sub-block's y (if fused), loaded here so the
    // loads land while the products below run: lane (lg, lc) reads 4
    // consecutive columns of token row lc (8 bytes; 16 lanes cover a 32-byte
    // row piece), and the identity product brings them into the layout of y.
    s16x4 gq[TB] = {};
    if (WITH_Y && p.gate) {
        const short* gp = static_cast<const short*>(p.gate);
        const int64_t g0 = (static_cast<int64_t>(b) * p.T + t0) * p.H + hd;
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
            gq[tb] = *reinterpret_cast<const s16x4*>(gp + (g0 + static_cast<int64_t>(16 * tb + lc) * p.H) * D + 16 * w + 4 * lg);
    }

    // ---- H = K Z - V for this wave's columns; |h|^2 partials; H to LDS ----
    f32x4 accH[TB];
    s16x4 hfh[TB], hfl[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
        f32x4 a = {0.f, 0.f, 0.f, 0.f};
        if (p.mode == 0) {
            if constexpr (G::K32_M) {
#pragma unroll
                for (int km = 0; km < M / 32; ++km) {
                    const bf16x8 kf = ld8(ks + (16 * tb + lc) * G::KS_LD + 32 * km + 8 * lg);
                    a = mma32(kf, z8l[km], a);
                    a = mma32(kf, z8h[km], a);
                }
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const s16x4 kf = *reinterpret_cast<const s16x4*>(ks + (16 * tb + lc) * G::KS_LD + 16 * mt + 4 * lg);
                    a = mma(kf, zfl[mt], a);
                    a = mma(kf, zfh[mt], a);
                }
            }
        }
        const float vsign = p.mode == 2 ? 1.f : -1.f;  // h = v for the encoding layer
#pragma unroll
        for (int r = 0; r < 4; ++r) a[r] = fmaf(vsign, bf16_val(vs[(16 * tb + 4 * lg + r) * G::VS_LD + dcol]), a[r]);
        accH[tb] = a;
        split4(a, hfh[tb], hfl[tb]);
        if constexpr (G::K32_C) {
            *reinterpret_cast<s16x4*>(hth + dcol * G::HT_LD + 16 * tb + 4 * lg) = hfh[tb];
            *reinterpret_cast<s16x4*>(htl + dcol * G::HT_LD + 16 * tb + 4 * lg) = hfl[tb];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * tb + 4 * lg + r;
            hsh[row * G::HS_LD + dcol] = hfh[tb][r];
            hsl[row * G::HS_LD + dcol] = hfl[tb][r];
        }
    }
    // |h_t|^2 partial sums over this wave's 16 columns: all reductions first,
    // then one guarded block of stores.
    {
        float sq[TB][4];
#pragma unroll
        for (int tb = 0; tb < TB; ++tb)
#pragma unroll
            for (int r = 0; r < 4; ++r) sq[tb][r] = row16_sum(accH[tb][r] * accH[tb][r]);
        if (lc == 0) {
#pragma unroll
            for (int tb = 0; tb < TB; ++tb)
#pragma unroll
                for (int r = 0; r < 4; ++r) hp[w * C0 + 16 * tb + 4 * lg + r] = sq[tb][r];
        }
    }
    __syncthreads();  // (A) H, |h|^2 partials visible

    // ---- c = H Z^T for this wave's slot tiles; gates in registers --------
#pragma unroll
    for (int mi = 0; mi < G::MPW; ++mi) {
        const int mb = w + mi * G::NW;
        if (mb < MT) {
            const int i = 16 * mb + lc;  // this lane's slot
            float gt[TB][4], kp[TB][4], tot[TB], ex_lo[TB], ex_hi[TB], first_rows = 1.f;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
                if constexpr (G::K32_D) {
#pragma unroll
                    for (int kd = 0; kd < D / 32; ++kd) {
                        const int ao = (16 * tb + lc) * G::HS_LD + 32 * kd + 8 * lg;
                        const int bo = (16 * mb + lc) * G::ZS_LD + 32 * kd + 8 * lg;
                        c = mma32x3(ld8(hsh + ao), ld8(hsl + ao), ld8(zh + bo), ld8(zl + bo), c);
                    }
                } else {
#pragma unroll
                    for (int kd = 0; kd < D / 16; ++kd) {
                        const int ao = (16 * tb + lc) * G::HS_LD + 16 * kd + 4 * lg;
                        const int bo = (16 * mb + lc) * G::ZS_LD + 16 * kd + 4 * lg;
                        c = mma3(*reinterpret_cast<const s16x4*>(hsh + ao), *reinterpret_cast<const s16x4*>(hsl + ao),
                                 *reinterpret_cast<const s16x4*>(zh + bo), *reinterpret_cast<const s16x4*>(zl + bo), c);
                    }
                }
                float prod = 1.f;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tau = 16 * tb + 4 * lg + r;
                    float hh = 0.f;
#pragma unroll
                    for (int ww = 0; ww < G::NW; ++ww) hh += hp[ww * C0 + tau];
                    const float k = bf16_val(ks[tau * G::KS_LD + i]);
                    const float mu = mus[tau];
                    // writing coefficient: k, or the encoding error c - k
                    const float a = bf16_val(gs[tau * G::GS_LD + i]) * (p.mode == 2 ? c[r] - k : k);
                    const float wv = fmaxf(fmaf(-c[r], c[r], hh), 0.f);
                    const float beta = __builtin_amdgcn_rsqf(fmaf(mu, mu, a * a * wv));
                    gt[tb][r] = beta * fmaf(a, c[r], mu);
                    kp[tb][r] = -beta * a;
                    prod *= gt[tb][r];
                }
                group_scan(prod, lg, ex_lo[tb], ex_hi[tb], tot[tb]);
                if (TB == 1) first_rows = rows01_prod(prod);
            }
            // Running (A, relative to a_ref) and suffix (prod_{l > t}) products
            // over the sub-block.
            const float aref = half_product<TB>(tot, first_rows);
            float fwd = 1.f / aref;
#pragma unroll
            for (int tb = 0; tb < TB; ++tb) {
                float bwd = 1.f;
#pragma unroll
                for (int tb2 = tb + 1; tb2 < TB; ++tb2) bwd *= tot[tb2];
                float A = fwd * ex_lo[tb];
                float suf[4];
                float s = bwd * ex_hi[tb];
#pragma unroll
                for (int r = 3; r >= 0; --r) {
                    suf[r] = s;
                    s *= gt[tb][r];
                }
                s16x4 wh4, wl4;
                split4(f32x4{kp[tb][0] * suf[0], kp[tb][1] * suf[1], kp[tb][2] * suf[2], kp[tb][3] * suf[3]}, wh4, wl4);
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int tau = 16 * tb + 4 * lg + r;
                    A *= gt[tb][r];
                    short hi, lo;
                    if constexpr (WITH_Y) {
                        split1(bf16_val(qs[tau * G::GS_LD + i]) * A, hi, lo);
                        qah[tau * G::QA_LD + i] = hi;
                        qal[tau * G::QA_LD + i] = lo;
                        split1(kp[tb][r] / A, hi, lo);
                        kah[tau * G::QA_LD + i] = hi;
                        kal[tau * G::QA_LD + i] = lo;
                    }
                }
                *reinterpret_cast<s16x4*>(wth + i * G::WT_LD + 16 * tb + 4 * lg) = wh4;
                *reinterpret_cast<s16x4*>(wtl + i * G::WT_LD + 16 * tb + 4 * lg) = wl4;
                fwd *= tot[tb];
            }
            if (lg == 0) {
                aend[i] = fwd * aref;
                arefs[i] = aref;
            }
        }
    }
    if (has_next) commit<G, WITH_Y>(nxt, st_next, p.gamma_per_slot != 0);
    __syncthreads();  // (B) W^T, A_end, Q.A, kappa/A and the next staged inputs visible

    // ---- read-out: Y = (Q.A) R + tril(P) H, P^T = (kappa/A)(Q.A)^T ---
    if constexpr (WITH_Y) {
        // R scaled by a_ref per slot (the Q.A tiles are relative to it)
        s16x4 rfh[MT], rfl[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const f32x4 ar = *reinterpret_cast<const f32x4*>(arefs + 16 * mt + 4 * lg);
            f32x4 rs = acc_R[mt];
#pragma unroll
            for (int r = 0; r < 4; ++r) rs[r] *= ar[r];
            split4(rs, rfh[mt], rfl[mt]);
        }
        const int64_t row0 = (static_cast<int64_t>(b) * p.T + t0) * p.H + hd;
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
            if (p.gate) {
                const f32x4 gf = tr16f(gq[tb], eye_operand(false));  // gate of tokens 16tb + 4lg + r, column dcol
#pragma unroll
                for (int r = 0; r < 4; ++r) y[r] *= gelu(gf[r]);
            }
#pragma unroll
            for (int r = 0; r < 4; ++r)
                st_y1(p.y, (row0 + static_cast<int64_t>(16 * tb + 4 * lg + r) * p.H) * D + dcol, y[r], p.y_bf16);
        }
    }

    // ---- state update: R <- diag(A_end) R + W^T H ----------------------
    if (need_state) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            f32x4 a = acc_R[mt];
#pragma unroll
            for (int r = 0; r < 4; ++r) a[r] *= aend[16 * mt + 4 * lg + r];
            if constexpr (G::K32_C) {
#pragma unroll
                for (int kt = 0; kt < C0 / 32; ++kt) {
                    const int ao = (16 * mt + lc) * G::WT_LD + 32 * kt + 8 * lg;
                    const int bo = dcol * G::HT_LD + 32 * kt + 8 * lg;
                    a = mma32x3(ld8(wth + ao), ld8(wtl + ao), ld8(hth + bo), ld8(htl + bo), a);
                }
            } else {
#pragma unroll
                for (int tb = 0; tb < TB; ++tb) {
                    const int ao = (16 * mt + lc) * G::WT_LD + 16 * tb + 4 * lg;
                    a = mma3(*reinterpret_cast<const s16x4*>(wth + ao), *reinterpret_cast<const s16x4*>(wtl + ao),
                             hfh[tb], hfl[tb], a);
                }
            }
            acc_R[mt] = a;
        }
    }
}

// Project every slot (row) of the accumulator-held state onto the unit
// sphere: sums of squares over each wave's 16 columns, then across waves.
template <int M, int D, class G>
__device__ __forceinline__ void project_state(f32x4 (&acc)[M / 16], char* smem) {
    float* np = reinterpret_cast<float*>(smem + G::O_NP);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, lc = lane & 15;
    // All row sums first (independent DPP chains the compiler can interleave),
    // then a single guarded block of stores.
    float ss[M / 16][4];
#pragma unroll
    for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) ss[mt][r] = row16_sum(acc[mt][r] * acc[mt][r]);
    if (lc == 0) {
#pragma unroll
        for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
            for (int r = 0; r < 4; ++r) np[w * M + 16 * mt + 4 * lg + r] = ss[mt][r];
    }
    __syncthreads();
#pragma unroll
    for (int mt = 0; mt < M / 16; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            float n2 = 0.f;
#pragma unroll
            for (int ww = 0; ww < D / 16; ++ww) n2 += np[ww * M + 16 * mt + 4 * lg + r];
            acc[mt][r] *= __builtin_amdgcn_rsqf(n2);
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

// Chunk-start state Z (in acc) -> B-operand fragments and the row-major LDS
// copy used by c = H Z^T.  The caller guarantees no wave still reads zh/zl.
template <int M, int D, class G>
__device__ __forceinline__ void stage_z(const f32x4 (&acc)[M / 16], s16x4 (&zfh)[M / 16], s16x4 (&zfl)[M / 16],
                                        bf16x8 (&z8h)[(M + 31) / 32], bf16x8 (&z8l)[(M + 31) / 32], char* smem) {
    short* zh = reinterpret_cast<short*>(smem + G::O_ZH);
    short* zl = reinterpret_cast<short*>(smem + G::O_ZL);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, lg = lane >> 4, lc = lane & 15;
#pragma unroll
    for (int mt = 0; mt < M / 16; ++mt) {
        split4(acc[mt], zfh[mt], zfl[mt]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int row = 16 * mt + 4 * lg + r;
            zh[row * G::ZS_LD + 16 * w + lc] = zfh[mt][r];
            zl[row * G::ZS_LD + 16 * w + lc] = zfl[mt][r];
        }
    }
    if constexpr (G::K32_M) {
        // B operands of H = K Z with k = slot: 8 consecutive slots of this
        // lane's column.  The column belongs to this wave, so its own LDS
        // writes above are all it reads (no barrier needed).
#pragma unroll
        for (int km = 0; km < M / 32; ++km)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int row = 32 * km + 8 * lg + j;
                z8h[km][j] = __builtin_bit_cast(__bf16, zh[row * G::ZS_LD + 16 * w + lc]);
                z8l[km][j] = __builtin_bit_cast(__bf16, zl[row * G::ZS_LD + 16 * w + lc]);
            }
    }
}

// Fused forward: one workgroup per (b, h), sequential over chunks, state
// passing and read-out together (no workspace).  Used when the (b, h)
// sequences alone fill the GPU.
template <int M, int D, int C0>
__global__ __launch_bounds__(4 * D) void osr_fused_kernel(Params p) {
    using G = Cfg<M, D, C0, true>;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    short* stage = reinterpret_cast<short*>(smem + G::O_KS);
    const int bh = blockIdx.x, b = bh / p.H, hd = bh % p.H;
    const int C = p.chunk, NS = p.T / C0, SPC = C / C0;
    f32x4 acc[G::MT];
    s16x4 zfh[G::MT], zfl[G::MT];
    bf16x8 z8h[(M + 31) / 32], z8l[(M + 31) / 32];
    Pre<G> nxt;
    const PreOff<G> poff = prefetch_offsets<G>(p);
    load_rows<M, D>(acc, p.state_in + static_cast<int64_t>(bh) * M * D);
    prefetch<G, true>(nxt, poff, p, b, hd, 0);
    commit<G, true>(nxt, stage, p.gamma_per_slot != 0);
    for (int s = 0; s < NS; ++s) {
        const int t0 = s * C0;
        // Unconditional (the last sub-block re-reads its own tile) so the
        // prefetch registers are never a conditionally written aggregate.
        const bool has_next = s + 1 < NS;
        if (s % SPC == 0) project_state<M, D, G>(acc, smem);  // its barriers also publish the first staged inputs
        prefetch<G, true>(nxt, poff, p, b, hd, has_next ? t0 + C0 : t0);
        if (s % SPC == 0) stage_z<M, D, G>(acc, zfh, zfl, z8h, z8l, smem);
        osr_subblock<M, D, C0, true>(p, smem, acc, zfh, zfl, z8h, z8l, s % SPC == 0, stage + (s & 1) * G::STAGE, nxt,
                                     stage + ((s + 1) & 1) * G::STAGE, has_next, true, b, hd, t0);
    }
    project_state<M, D, G>(acc, smem);
    store_rows<M, D>(acc, p.state_out + static_cast<int64_t>(bh) * M * D);
}

}  // namespace mfma
}  // namespace osr
