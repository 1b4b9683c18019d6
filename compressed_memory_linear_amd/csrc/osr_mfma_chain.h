// osr_mfma_chain.h -- inter-chunk state passing of the chunk-wise OSR forward
// on gfx950 matrix cores.
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646), section "Parallel and Hardware Efficient Form", eq.
// recurrence_linear2: inside a chunk every projection, gate and h_t is taken at
// the unit-projected chunk-start state Z, so the chunk-end state is
//   R_end = diag(A_C) Z + sum_t diag(kappa_t (.) prod_{l > t} g_l) 1 h_t^T
// with H = K Z - V (decoding) or -V (similarity), c = H Z^T,
// a = gamma (.) k, w = max(|h|^2 - c^2, 0), beta = (mu^2 + a^2 w)^(-1/2)
// (appendix "Computing beta"), g = beta (mu + a c), kappa = -beta a.  This
// kernel carries that state from chunk to chunk (one workgroup per (b, h),
// sequential over chunks) and stores, per chunk, Z, the gates g and kappa and
// the vectors h_t, from which the read-out kernel forms every y_t in parallel
// over chunks.
//
// Work layout (transposed relative to the read-out kernels): one workgroup of
// m/16 waves; wave w owns the slot rows [16w, 16w + 16) of the state for all d
// columns, held as MFMA accumulator tiles of R^T (lane (lg, lc) of tile j
// holds R[16w + lc][16j + 4lg + r]).  With that ownership
//   * the per-slot projection onto the unit sphere is wave-local;
//   * the tiles of Z^T are, as they stand, B operands of c = H Z^T for the
//     wave's own slots, whose gates the same wave forms;
//   * the gated suffix products W (tokens x slots) come out of the gate phase
//     already in the B-operand layout of the update R^T += H^T W, and A_end is
//     a per-lane scalar;
// so a sub-block needs one workgroup barrier after H is written (plus one at
// its start that publishes Z, the staged inputs and frees the H buffers).
// H = K Z - V contracts over slots, which span all waves: Z^T goes through
// LDS once per chunk and the H tiles are shared through LDS in both the
// token-major (for c) and the column-major (for the update) layout.
//
// Split over P workgroups (P > 1; few sequences, so the chip is otherwise
// idle).  Inside a chunk the gates, h_t and the update of a group of tokens
// depend only on Z and that group's inputs, and the update is linear in the
// state: with U_p = sum over sub-block p of diag(kappa_t (.) prod_{l > t,
// l in p} g_l) 1 h_t^T and t_p the product of g over sub-block p,
//   R_end = diag(t_0 ... t_{P-1}) Z + sum_p diag(t_{p+1} ... t_{P-1}) U_p.
// Workgroup p takes sub-block p of every chunk: it forms H, c, the gates, the
// workspace entries, U_p and t_p for its tokens, publishes (U_p, t_p), reads
// the other workgroups' and forms R_end; every workgroup holds the same Z.
// The hand-off goes through device memory with agent-scope (coherent across
// XCDs) accesses: the data, then a completion counter once the data stores
// have retired; readers wait for the counter (a bounded wait), then read.
// Consecutive chunks use alternate buffers; a workgroup reuses a buffer only
// after every workgroup has read it (it has seen their next counters).
//
// 16x16x32 operands built from accumulator tiles use a permuted k order: two
// D-layout tiles t0, t1 (lane (lg, lc) holds rows 4lg..4lg+3 of column lc)
// concatenated form a B operand whose k index 8lg + j stands for row
// 16(j/4) + 4lg + j%4 of the 32-row block; the matching A operand is read from
// LDS as two 8-byte pieces at columns 4lg and 16 + 4lg of the block.  Any
// bijection of k leaves the contraction unchanged.
#pragma once

#include "osr_mfma_kernels.h"

namespace osr {
namespace mfma {

// PAIR: two waves per slot block (one group of m/16 waves per token half of
// the chunk); see osr_chain_kernel.
template <int M, int D, int C0, bool PAIR = false>
struct ChainCfg {
    static constexpr int M_ = M, D_ = D, C0_ = C0;
    static constexpr int NWS = M / 16;        // slot blocks; wave w owns slots [16(w%NWS), +16)
    static constexpr int NG = PAIR ? 2 : 1;   // wave groups, each over C0/NG tokens
    static constexpr int NW = NG * NWS;
    static constexpr int NT = 64 * NW;
    static constexpr int DB = D / 16;   // column tiles
    static constexpr int TB = C0 / 16;  // token tiles per sub-block
    static constexpr int TBW = TB / NG; // token tiles per group
    // H = K Z - V work split inside a group: TG waves take distinct token
    // tiles, and the WS waves that share a token tile split its column tiles;
    // WSE of those have work (WSE partial |h|^2 sums per token).
    static constexpr int TG = TBW < NWS ? TBW : NWS;
    static constexpr int WS = NWS / TG;
    static constexpr int WSE = WS < DB ? WS : DB;
    static constexpr int TPW = TBW / TG;  // token tiles per wave
    static constexpr int DPW = DB / WSE;  // column tiles per wave
    // Row strides (bf16 elements).  Buffers read as 16-byte MFMA operands
    // (rows lc = 0..15) pad by 8: a stride of 4 (mod 8) words puts the 8 lanes
    // of a 128-byte read phase on distinct bank quads.  The H buffers, read as
    // 8-byte operands and written as scattered 2-byte rows 4lg + r, pad by 4:
    // a stride of 2 (mod 4) words makes both conflict-free.
    static constexpr int ZT_LD = M + 8;
    static constexpr int KS_LD = M + 8;
    static constexpr int VS_LD = D + 8;
    static constexpr int HS_LD = D + 4;
    static constexpr int HT_LD = C0 + 4;
    static constexpr int GS_LD = M + 8;
    static constexpr bool K32_M = M % 32 == 0;      // H = K Z     (k = slot)
    static constexpr bool K32_D = D % 32 == 0;      // c = H Z^T   (k = column)
    static constexpr bool K32_C = TBW % 2 == 0;     // R^T += H^T W (k = token, a group's tokens)
    // Staged inputs, as in the read-out kernels (no q).
    static constexpr int KPC = C0 * M / 8, KPT = (KPC + NT - 1) / NT;
    static constexpr int VPC = C0 * D / 8, VPT = (VPC + NT - 1) / NT;
    static constexpr int SO_K = 0;
    static constexpr int SO_V = SO_K + C0 * KS_LD;
    static constexpr int SO_G = SO_V + C0 * VS_LD;
    static constexpr int SO_Q = SO_G + C0 * GS_LD;
    static constexpr int SO_MU = SO_Q;           // mu [C0] fp32
    static constexpr int STAGE = SO_MU + 2 * C0;
    // LDS layout (bytes).
    static constexpr int O_ZTH = 0;                          // Z^T hi [D][ZT_LD]
    static constexpr int O_ZTL = O_ZTH + D * ZT_LD * 2;      // Z^T lo
    static constexpr int O_KS = O_ZTL + D * ZT_LD * 2;       // staging [2][STAGE]
    static constexpr int O_HH = O_KS + 2 * STAGE * 2;        // H hi   [C0][HS_LD]
    static constexpr int O_HL = O_HH + C0 * HS_LD * 2;       // H lo
    static constexpr int O_TH = O_HL + C0 * HS_LD * 2;       // H^T hi [D][HT_LD]
    static constexpr int O_TL = O_TH + D * HT_LD * 2;        // H^T lo
    static constexpr int O_HP = O_TL + D * HT_LD * 2;        // |h|^2 partials [C0][WSE]
    static constexpr int O_XU = O_HP + C0 * WSE * 4;         // pair exchange: U [NW][64 lanes][DB] f32x4
    static constexpr int O_XT = O_XU + (PAIR ? NW * 64 * DB * 16 : 0);  // and the half products [NW][64]
    static constexpr int BYTES = O_XT + (PAIR ? NW * 64 * 4 : 0);

    static_assert(M % 16 == 0 && D % 16 == 0 && C0 % 16 == 0, "tile multiples");
    static_assert(TB % NG == 0, "token tiles split evenly between the groups");
    static_assert(NT <= 1024, "waves");
};

template <int M, int D, int C0, bool PAIR = false>
constexpr bool chain_fits() {
    return ChainCfg<M, D, C0, PAIR>::BYTES <= 160 * 1024;
}

// Unit-sphere projection of the wave's slot rows (eq. normalized_recurrence):
// lane (lg, lc) holds 4 columns of slot lc per tile; the row sum adds the
// four lane rows.
template <int DB>
__device__ __forceinline__ float row_inv_norm(const f32x4 (&acc)[DB]) {
    float n2 = 0.f;
#pragma unroll
    for (int j = 0; j < DB; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) n2 = fmaf(acc[j][r], acc[j][r], n2);
    return __builtin_amdgcn_rsqf(rows4_sum(n2));
}

// ONE: one sub-block per chunk (C0 = C), known at compile time so the
// chunk-start work is straight-line code.
// PAIR (requires ONE): two waves per slot block, group g = 0, 1 of m/16 waves
// taking the chunk's token half g.  Inside a chunk every gate depends only on
// Z and the inputs, so the halves are independent except for the suffix
// products that cross from half 0 into half 1: with U_g = sum over half g of
// kappa_t (.) (prod of g_l over l > t within half g) h_t^T and t_g the
// per-slot product of the gates over half g,
//   R_end = diag(t_0 t_1) Z + diag(t_1) U_0 + U_1.
// Each wave of a pair forms its U_g and t_g, the pair swaps them through
// LDS, and both form R_end (and its projection) identically.  This doubles
// the waves per SIMD (latency hiding) at one extra barrier per chunk.
// ENC: the encoding layer (h = v, writing coefficient c - k), a separate
// instantiation so that the other objectives carry none of its selects.
// LIN1: the first chunk linearisation (eq. recurrence_linear1): gate mu beta
// and a term e Z with e = beta a c on the chunk-start slots, so that
//   R_end = diag(A_end) R + diag(sum_t e_t (.) prod_{l > t} g_l) Z + H^T W
// (the coefficient of Z is summed alongside W); e goes to the workspace too.
// RAW: also store, for the backward, every chunk-start state before projection
// and the end state (Params::raw) and c, beta, |h|^2 of every token
// (Params::raw_c, raw_b, raw_hh); its own instantiation, so the forward carries
// none of it.
// Floats of one workgroup's hand-off: U_p as [wave][column tile][lane] f32x4,
// then t_p as [wave][lane].
template <int M, int D>
constexpr int64_t xchg_floats() {
    return static_cast<int64_t>(M / 16) * (D / 16) * 64 * 4 + (M / 16) * 64;
}
// Progress counters of the hand-off: one per (sequence, workgroup, wave),
// XFLAG_STRIDE ints apart (XFLAG_STRIDE, XSPIN, XCPOL_SC1, xrsrc: osr_device.h).
// Wait until wave w of workgroup q of sequence bh has published chunk s
// (its counter passed s); gives up after XSPIN polls (broken = true).
template <class G>
__device__ __forceinline__ void xwait(const Params& p, int bh, int P, int q, int w, int s, bool& broken) {
    const int* f = p.xflags + ((bh * P + q) * G::NWS + w) * XFLAG_STRIDE;
    int n = 0;
    while (__hip_atomic_load(const_cast<int*>(f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <= s) {
        if (++n >= XSPIN) {
            broken = true;
            break;
        }
    }
}

template <int M, int D, int C0, bool WRITE_Z, bool ONE, bool PAIR, bool ENC, bool LIN1 = false, bool RAW = false,
          int P = 1>
__global__ __launch_bounds__(4 * M * (PAIR ? 2 : 1)) void osr_chain_kernel(Params p) {
    using G = ChainCfg<M, D, C0, PAIR>;
    static_assert(!PAIR || ONE, "the pair split covers one sub-block per chunk");
    static_assert(P == 1 || (!ONE && !PAIR && !RAW), "the workgroup split takes one sub-block per workgroup");
    constexpr int DB = G::DB, TBW = G::TBW;
    __shared__ __attribute__((aligned(16))) char smem[G::BYTES];
    short* stage = reinterpret_cast<short*>(smem + G::O_KS);
    short* zth = reinterpret_cast<short*>(smem + G::O_ZTH);
    short* ztl = reinterpret_cast<short*>(smem + G::O_ZTL);
    short* hsh = reinterpret_cast<short*>(smem + G::O_HH);
    short* hsl = reinterpret_cast<short*>(smem + G::O_HL);
    short* hth = reinterpret_cast<short*>(smem + G::O_TH);
    short* htl = reinterpret_cast<short*>(smem + G::O_TL);
    float* hp = reinterpret_cast<float*>(smem + G::O_HP);

    // P > 1: the P workgroups of a sequence are 8 block indices apart, so the
    // round-robin dispatch puts them on one XCD (correctness does not depend
    // on it); blocks past the last sequence exit at once.
    int bh = blockIdx.x, pidx = 0;
    if constexpr (P > 1) {
        pidx = (blockIdx.x / 8) % P;
        bh = blockIdx.x % 8 + 8 * (blockIdx.x / (8 * P));
        if (bh >= p.B * p.H) return;
    }
    const int b = bh / p.H, hd = bh % p.H;
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const int lg = lane >> 4, lc = lane & 15;
    const int grp = PAIR ? w / G::NWS : 0;  // token half of this wave
    const int wv = w % G::NWS;              // slot block of this wave
    const int slot = 16 * wv + lc;
    const int tbg = grp * TBW;              // first token tile of the group
    const int C = p.chunk, SPC = C / C0, NC = p.T / C;
    // chunk range [n0, n1): iterations s over chunks (P > 1) or sub-blocks
    const int n0 = p.n_begin, n1 = p.n_end > 0 ? p.n_end : NC;
    const int S0 = P > 1 ? n0 : n0 * SPC, NS = P > 1 ? n1 : n1 * SPC;
    bool xbroken = false;  // a hand-off wait gave up: stop waiting (the results are then wrong)
    // H = K Z - V assignment of this wave (inside its group).
    const int g1_tb0 = tbg + wv % G::TG, g1_grp = wv / G::TG;
    const bool g1_active = g1_grp < G::WSE;
    const s16x4 eye = eye_operand(false), neg_eye = eye_operand(true);

    f32x4 acc[DB];             // R^T tiles: acc[j][r] = R[slot][16j + 4lg + r]
    s16x4 zfh[DB], zfl[DB];    // split Z^T tiles: B operands of c = H Z^T
    Pre<G> nxt;

    {
        // the initial state, or the unprojected state a previous chunk range handed on
        const float* src = (n0 > 0 ? p.carry : p.state_in) + static_cast<int64_t>(bh) * M * D +
                           static_cast<int64_t>(slot) * D + 4 * lg;
#pragma unroll
        for (int j = 0; j < DB; ++j) acc[j] = *reinterpret_cast<const f32x4*>(src + 16 * j);
    }
    const PreOff<G> poff = prefetch_offsets<G>(p);
    prefetch<G, false>(nxt, poff, p, b, hd, n0 * C + pidx * C0);
    commit<G, false>(nxt, stage, p.gamma_per_slot != 0);
    // Drain the loads above before the loop.  Left pending, they make the
    // compiler's wait analysis treat the loop-carried state tiles as possibly
    // still in flight at the loop head, and it then waits there for every
    // memory operation of the previous sub-block, stores included.
    __builtin_amdgcn_s_waitcnt(0);

    for (int s = S0; s < NS; ++s) {
        // P > 1: iteration s is chunk s, this workgroup's sub-block pidx of it
        const int t0 = P > 1 ? s * C + pidx * C0 : s * C0;
        const bool chunk_start = ONE || P > 1 || s % SPC == 0;
        const int chunk = ONE || P > 1 ? s : s / SPC;
        const bool has_next = s + 1 < NS;
        const short* st = stage + ((s - S0) & 1) * G::STAGE;
        const short* ks = st + G::SO_K;
        const short* vs = st + G::SO_V;
        const short* gs = st + G::SO_G;
        const float* mus = reinterpret_cast<const float*>(st + G::SO_MU);
        // this sub-block's part of the chunk's workspace (read-out inputs)
        const Workspace ws = workspace_at<M, D>(p, bh, chunk);
        const int tc0 = ONE ? 0 : P > 1 ? pidx * C0 : (s % SPC) * C0;

        if (chunk_start) {
            if (RAW && grp == 0) {
                // the chunk-start state before projection, for the backward
                float* dst = p.raw + bh * p.raw_stride + static_cast<int64_t>(chunk) * M * D +
                             static_cast<int64_t>(slot) * D + 4 * lg;
#pragma unroll
                for (int j = 0; j < DB; ++j) *reinterpret_cast<f32x4*>(dst + 16 * j) = acc[j];
            }
            const float inv = row_inv_norm<DB>(acc);
#pragma unroll
            for (int j = 0; j < DB; ++j)
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[j][r] *= inv;
        }
        // Loads of the next sub-block, issued before this sub-block's
        // workspace stores (the memory counter retires in order).
        // Unconditional: the last sub-block re-reads its own tile.
        prefetch<G, false>(nxt, poff, p, b, hd, has_next ? t0 + (P > 1 ? C : C0) : t0);
        if (chunk_start) {
            // Z^T to LDS (read by every wave's H = K Z); the split tiles stay
            // in registers.  No wave reads Z^T between the last sub-block's
            // barrier (A) and the barrier (S) below.  A pair writes the hi
            // (group 0) and lo (group 1) halves.
#pragma unroll
            for (int j = 0; j < DB; ++j) {
                split4(acc[j], zfh[j], zfl[j]);
                // transposed, the lane holds slots 16wv + 4lg .. +3 of column 16j + lc
                const int zo = (16 * j + lc) * G::ZT_LD + 16 * wv + 4 * lg;
                if (!PAIR || grp == 0) *reinterpret_cast<s16x4*>(zth + zo) = tr16(zfh[j], eye);
                if (!PAIR || grp == 1) *reinterpret_cast<s16x4*>(ztl + zo) = tr16(zfl[j], eye);
            }
        }
        __syncthreads();  // (S) Z^T and this sub-block's staged inputs visible; H buffers free

        // ---- H = K Z - V (token tiles x column tiles of this wave) -------
        // Operands first, then the MFMAs of all tiles interleaved (independent
        // accumulators), then the epilogue.
        if (g1_active) {
            constexpr int TPW = G::TPW, DPW = G::DPW;
            // -V (+V for the encoding layer, whose h is v): rows of V read 8
            // bytes at a time and brought into the accumulator layout by the
            // (negated) identity on the 16-deep matrix core.  Where K Z runs
            // on the 32-deep form, its chain starts from zero and -V is added
            // on the VALU afterwards, so no 16-deep result is ever the
            // accumulator input of a 32-deep product (no shared accumulator
            // between the two shapes anywhere in this kernel).
            const s16x4 v_eye = ENC ? eye : neg_eye;
            f32x4 ha[TPW][DPW], vt[TPW][DPW];
#pragma unroll
            for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
                for (int dj = 0; dj < DPW; ++dj) {
                    const int tb = g1_tb0 + G::TG * ti, dc0 = 16 * (g1_grp + G::WSE * dj);
                    vt[ti][dj] = tr16f(ld4s(vs + (16 * tb + lc) * G::VS_LD + dc0 + 4 * lg), v_eye);
                    ha[ti][dj] = (G::K32_M && p.mode == 0) ? f32x4{0.f, 0.f, 0.f, 0.f} : vt[ti][dj];
                }
            if (p.mode == 0) {
                if constexpr (G::K32_M) {
                    constexpr int KM = M / 32;
                    bf16x8 kf[TPW][KM];
#pragma unroll
                    for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
                        for (int km = 0; km < KM; ++km)
                            kf[ti][km] = ld8(ks + (16 * (g1_tb0 + G::TG * ti) + lc) * G::KS_LD + 32 * km + 8 * lg);
#pragma unroll
                    for (int km = 0; km < KM; ++km) {
                        bf16x8 zh8[DPW], zl8[DPW];
#pragma unroll
                        for (int dj = 0; dj < DPW; ++dj) {
                            const int zo = (16 * (g1_grp + G::WSE * dj) + lc) * G::ZT_LD + 32 * km + 8 * lg;
                            zh8[dj] = ld8(zth + zo);
                            zl8[dj] = ld8(ztl + zo);
                        }
#pragma unroll
                        for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
                            for (int dj = 0; dj < DPW; ++dj) ha[ti][dj] = mma32(kf[ti][km], zl8[dj], ha[ti][dj]);
#pragma unroll
                        for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
                            for (int dj = 0; dj < DPW; ++dj) ha[ti][dj] = mma32(kf[ti][km], zh8[dj], ha[ti][dj]);
                    }
#pragma unroll
                    for (int ti = 0; ti < TPW; ++ti)
#pragma unroll
                        for (int dj = 0; dj < DPW; ++dj) ha[ti][dj] += vt[ti][dj];
                } else {
                    s16x4 kf[TPW];
#pragma unroll
                    for (int ti = 0; ti < TPW; ++ti)
                        kf[ti] = ld4s(ks + (16 * (g1_tb0 + G::TG * ti) + lc) * G::KS_LD + 4 * lg);
#pragma unroll
                    for (int dj = 0; dj < DPW; ++dj) {
                        const int zo = (16 * (g1_grp + G::WSE * dj) + lc) * G::ZT_LD + 4 * lg;
                        const s16x4 zh4 = ld4s(zth + zo), zl4 = ld4s(ztl + zo);
#pragma unroll
                        for (int ti = 0; ti < TPW; ++ti) {
                            ha[ti][dj] = mma(kf[ti], zl4, ha[ti][dj]);
                            ha[ti][dj] = mma(kf[ti], zh4, ha[ti][dj]);
                        }
                    }
                }
            }
#pragma unroll
            for (int ti = 0; ti < TPW; ++ti) {
                const int tb = g1_tb0 + G::TG * ti;
                float sq[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int dj = 0; dj < DPW; ++dj) {
                    const int dcol = 16 * (g1_grp + G::WSE * dj) + lc;
                    const f32x4 a = ha[ti][dj];
                    if constexpr (WRITE_Z)
                        *reinterpret_cast<f32x4*>(ws.h + ws_frag(g1_grp + G::WSE * dj, tc0 / 16 + tb, C / 16, lane)) = a;
                    s16x4 hh4, hl4;
                    split4(a, hh4, hl4);
                    *reinterpret_cast<s16x4*>(hth + dcol * G::HT_LD + 16 * tb + 4 * lg) = hh4;
                    *reinterpret_cast<s16x4*>(htl + dcol * G::HT_LD + 16 * tb + 4 * lg) = hl4;
                    // token-major copy: transposed, the lane holds columns
                    // dcol - lc + 4lg .. +3 of token 16tb + lc
                    const int so = (16 * tb + lc) * G::HS_LD + dcol - lc + 4 * lg;
                    *reinterpret_cast<s16x4*>(hsh + so) = tr16(hh4, eye);
                    *reinterpret_cast<s16x4*>(hsl + so) = tr16(hl4, eye);
#pragma unroll
                    for (int r = 0; r < 4; ++r) sq[r] = fmaf(a[r], a[r], sq[r]);
                }
                // |h_t|^2 over this wave's columns: reductions first, one
                // guarded block of stores.
#pragma unroll
                for (int r = 0; r < 4; ++r) sq[r] = row16_sum(sq[r]);
                if (lc == 0) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) hp[(16 * tb + 4 * lg + r) * G::WSE + g1_grp] = sq[r];
                }
            }
        }
        __syncthreads();  // (A) H, H^T and |h|^2 partials visible

        // Z to the workspace, here rather than at the chunk start: there the
        // stores queue behind the prefetch loads on the way to barrier (S).
        // Stored as its bf16 hi/lo split (the operands every product of this
        // chunk used), transposed to the read-out kernel's accumulator layout
        // (slots 16wv + 4lg .. +3 of column 16j + lc), one 16-byte piece per
        // lane and tile.
        if constexpr (WRITE_Z) {
            if (chunk_start && grp == 0 && wv % P == pidx) {  // split: each workgroup stores some slot blocks
#pragma unroll
                for (int j = 0; j < DB; ++j) {
                    const s16x4 th = tr16(zfh[j], eye), tl = tr16(zfl[j], eye);
                    *reinterpret_cast<s16x8*>(ws.z + z_frag<D>(wv, j, lane)) =
                        __builtin_shufflevector(th, tl, 0, 1, 2, 3, 4, 5, 6, 7);
                }
            }
        }
        // ---- c = H Z^T for this wave's slots and its group's tokens; gates --
        // Gate inputs are read before the products.  Tile i of the group is
        // token tile tbg + i of the sub-block.
        constexpr bool enc = ENC;
        float hh[TBW][4], av[TBW][4], muv[TBW][4];
#pragma unroll
        for (int i = 0; i < TBW; ++i) {
            const int tb = tbg + i;
            if constexpr (G::WSE == 1) {
                const f32x4 h4 = *reinterpret_cast<const f32x4*>(hp + 16 * tb + 4 * lg);
#pragma unroll
                for (int r = 0; r < 4; ++r) hh[i][r] = h4[r];
            } else if constexpr (G::WSE % 4 == 0) {
                // WSE partials per token, contiguous: 16-byte broadcast reads.
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const f32x4* q4 = reinterpret_cast<const f32x4*>(hp + (16 * tb + 4 * lg + r) * G::WSE);
                    f32x4 x = q4[0];
#pragma unroll
                    for (int g = 1; g < G::WSE / 4; ++g) x += q4[g];
                    hh[i][r] = (x[0] + x[1]) + (x[2] + x[3]);
                }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const float* q4 = hp + (16 * tb + 4 * lg + r) * G::WSE;
                    float x = 0.f;
#pragma unroll
                    for (int g = 0; g < G::WSE; ++g) x += q4[g];
                    hh[i][r] = x;
                }
            }
            const f32x4 mu4 = *reinterpret_cast<const f32x4*>(mus + 16 * tb + 4 * lg);
            // k and gamma of tokens 16tb + 4lg + r for this lane's slot, from
            // 8-byte row reads brought into the accumulator layout
            const f32x4 k4 = tr16f(ld4s(ks + (16 * tb + lc) * G::KS_LD + 16 * wv + 4 * lg), eye);
            const f32x4 g4 = tr16f(ld4s(gs + (16 * tb + lc) * G::GS_LD + 16 * wv + 4 * lg), eye);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                // the encoding layer writes with gamma (c - k): keep -gamma k
                // here and add gamma c once c is known
                av[i][r] = enc ? -g4[r] * k4[r] : g4[r] * k4[r];
                muv[i][r] = mu4[r];
            }
        }
        // Tile-major: the products of token tile i are issued before the gates
        // of tile i - 1, so the gate arithmetic (VALU) of one tile can run under
        // the matrix-core products of the next.
        f32x4 cc[TBW];
        float gt[TBW][4], kp[TBW][4], ev[TBW][4], tot[TBW], ex_lo[TBW], ex_hi[TBW];
        auto gates = [&](int i) {
            float prod = 1.f;
            f32x4 bsave;  // beta of the tile's tokens (kept for the backward)
            f32x4 g4 = {0.f, 0.f, 0.f, 0.f};  // gamma of the tile, read again for the encoding layer only
            if (enc) g4 = tr16f(ld4s(gs + (16 * (tbg + i) + lc) * G::GS_LD + 16 * wv + 4 * lg), eye);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float mu = muv[i][r], cr = cc[i][r];
                const float a = enc ? fmaf(g4[r], cr, av[i][r]) : av[i][r];
                const float wvv = fmaxf(fmaf(-cr, cr, hh[i][r]), 0.f);
                const float beta = __builtin_amdgcn_rsqf(fmaf(mu, mu, a * a * wvv));
                bsave[r] = beta;
                if constexpr (LIN1) {
                    gt[i][r] = beta * mu;
                    ev[i][r] = beta * a * cr;
                } else {
                    gt[i][r] = beta * fmaf(a, cr, mu);
                }
                kp[i][r] = -beta * a;
                prod *= gt[i][r];
            }
            rows4_prod_scan(prod, lg, ex_lo[i], ex_hi[i], tot[i]);
            if constexpr (RAW) {
                // c, beta and |h|^2 of these tokens, for the backward
                const int64_t ch = static_cast<int64_t>(bh) * (p.T / C) + chunk;
                const int64_t o = ch * M * C + ws_frag(wv, tc0 / 16 + tbg + i, C / 16, lane);
                *reinterpret_cast<f32x4*>(p.raw_c + o) = cc[i];
                *reinterpret_cast<f32x4*>(p.raw_b + o) = bsave;
                if (wv == 0 && lc == 0) {
                    float* dst = p.raw_hh + ch * C + tc0 + 16 * (tbg + i) + 4 * lg;
#pragma unroll
                    for (int r = 0; r < 4; ++r) dst[r] = hh[i][r];
                }
            }
            if constexpr (WRITE_Z) {
                const int64_t o = ws_frag(wv, tc0 / 16 + tbg + i, C / 16, lane);
                *reinterpret_cast<f32x4*>(ws.g + o) = f32x4{gt[i][0], gt[i][1], gt[i][2], gt[i][3]};
                *reinterpret_cast<f32x4*>(ws.k + o) = f32x4{kp[i][0], kp[i][1], kp[i][2], kp[i][3]};
                if constexpr (LIN1)
                    *reinterpret_cast<f32x4*>(ws.e + o) = f32x4{ev[i][0], ev[i][1], ev[i][2], ev[i][3]};
            }
        };
        if constexpr (G::K32_D) {
            constexpr int KD = D / 32;
            bf16x8 bhk[KD], blk[KD];
#pragma unroll
            for (int kd = 0; kd < KD; ++kd) {
                bhk[kd] = cat8(zfh[2 * kd], zfh[2 * kd + 1]);
                blk[kd] = cat8(zfl[2 * kd], zfl[2 * kd + 1]);
            }
            auto products = [&](int i) {
                bf16x8 ah[KD], al[KD];
#pragma unroll
                for (int kd = 0; kd < KD; ++kd) {
                    const int ao = (16 * (tbg + i) + lc) * G::HS_LD + 32 * kd + 4 * lg;
                    ah[kd] = ld8p(hsh + ao);
                    al[kd] = ld8p(hsl + ao);
                }
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int kd = 0; kd < KD; ++kd) {
                    c = mma32(al[kd], bhk[kd], c);
                    c = mma32(ah[kd], blk[kd], c);
                    c = mma32(ah[kd], bhk[kd], c);
                }
                cc[i] = c;
            };
            products(0);
#pragma unroll
            for (int i = 1; i < TBW; ++i) {
                products(i);
                gates(i - 1);
            }
            gates(TBW - 1);
        } else {
#pragma unroll
            for (int i = 0; i < TBW; ++i) {
                const int ao = (16 * (tbg + i) + lc) * G::HS_LD + 4 * lg;
                cc[i] = mma3(ld4s(hsh + ao), ld4s(hsl + ao), zfh[0], zfl[0], f32x4{0.f, 0.f, 0.f, 0.f});
            }
#pragma unroll
            for (int i = 0; i < TBW; ++i) gates(i);
        }
        // W_t = kappa_t (.) prod_{l > t} g_l over the group's tokens, split into
        // B operands of the update (k = token); aend = prod of the group's g.
        s16x4 wh4[TBW], wl4[TBW];
        float aend = 1.f, ez = 0.f;  // ez (LIN1): the lane's part of the coefficient of Z
#pragma unroll
        for (int i = TBW - 1; i >= 0; --i) {
            float s_ = aend * ex_hi[i];
            f32x4 wvec;
#pragma unroll
            for (int r = 3; r >= 0; --r) {
                wvec[r] = kp[i][r] * s_;
                if constexpr (LIN1) ez = fmaf(ev[i][r], s_, ez);
                s_ *= gt[i][r];
            }
            split4(wvec, wh4[i], wl4[i]);
            aend *= tot[i];
        }
        if constexpr (LIN1) ez = rows4_sum(ez);

        // ---- R^T <- R^T diag(A_end) + H^T W (PAIR: U_g = H^T W over half g) --
        f32x4 u[DB];
#pragma unroll
        for (int db = 0; db < DB; ++db) {
            if constexpr (LIN1) {
                // Z: the running state itself when a chunk is one sub-block
                // (or with the workgroup split, where acc holds Z), else its
                // split (hi + lo) kept from the chunk start
                f32x4 zf = acc[db];
                if constexpr (!ONE && P == 1) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) zf[r] = bf16_bits_to_f32(static_cast<uint16_t>(zfh[db][r])) +
                                                      bf16_bits_to_f32(static_cast<uint16_t>(zfl[db][r]));
                }
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    u[db][r] = PAIR || P > 1 ? zf[r] * ez : fmaf(acc[db][r], aend, zf[r] * ez);
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) u[db][r] = PAIR || P > 1 ? 0.f : acc[db][r] * aend;
            }
        }
        if constexpr (G::K32_C) {
#pragma unroll
            for (int kt = 0; kt < TBW / 2; ++kt) {
                bf16x8 th[DB], tl[DB];
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int ao = (16 * db + lc) * G::HT_LD + 16 * tbg + 32 * kt + 4 * lg;
                    th[db] = ld8p(hth + ao);
                    tl[db] = ld8p(htl + ao);
                }
                const bf16x8 bh = cat8(wh4[2 * kt], wh4[2 * kt + 1]), bl = cat8(wl4[2 * kt], wl4[2 * kt + 1]);
#pragma unroll
                for (int db = 0; db < DB; ++db) u[db] = mma32(tl[db], bh, u[db]);
#pragma unroll
                for (int db = 0; db < DB; ++db) u[db] = mma32(th[db], bl, u[db]);
#pragma unroll
                for (int db = 0; db < DB; ++db) u[db] = mma32(th[db], bh, u[db]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < TBW; ++i)
#pragma unroll
                for (int db = 0; db < DB; ++db) {
                    const int ao = (16 * db + lc) * G::HT_LD + 16 * (tbg + i) + 4 * lg;
                    u[db] = mma3(ld4s(hth + ao), ld4s(htl + ao), wh4[i], wl4[i], u[db]);
                }
        }

        // Next sub-block's inputs into the other staging buffer (its last
        // readers, the previous sub-block's gates, finished before (S)).
        // The memory counter retires loads and stores in order; the loads
        // were issued before this sub-block's workspace stores, so the wait
        // for them here leaves those stores in flight.
        if (has_next) commit<G, false>(nxt, stage + ((s + 1 - S0) & 1) * G::STAGE, p.gamma_per_slot != 0);

        if constexpr (PAIR) {
            // Swap (U_g, t_g) within the pair; both form
            // R_end = diag(t_0 t_1) Z + diag(t_1) U_0 + U_1 (acc holds Z).
            f32x4* xu = reinterpret_cast<f32x4*>(smem + G::O_XU);
            float* xt = reinterpret_cast<float*>(smem + G::O_XT);
#pragma unroll
            for (int db = 0; db < DB; ++db) xu[(w * 64 + lane) * DB + db] = u[db];
            xt[w * 64 + lane] = aend;
            __syncthreads();  // (X) both halves' U and t visible
            const int pw = (1 - grp) * G::NWS + wv;  // partner wave
            const float tp = xt[pw * 64 + lane];
            const float t0h = grp == 0 ? aend : tp, t1h = grp == 0 ? tp : aend;
            const float az = t0h * t1h;
#pragma unroll
            for (int db = 0; db < DB; ++db) {
                const f32x4 up = xu[(pw * 64 + lane) * DB + db];
                const f32x4 u0 = grp == 0 ? u[db] : up, u1 = grp == 0 ? up : u[db];
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[db][r] = fmaf(acc[db][r], az, fmaf(u0[r], t1h, u1[r]));
            }
        } else if constexpr (P > 1) {
            // Publish (U_p, t_p), then R_end = diag(prod_q t_q) Z +
            // sum_q diag(prod_{q' > q} t_q') U_q by Horner's rule in q order,
            // R <- R (.) t_q + U_q from R = Z, with the same operations in the
            // same order in every workgroup (so all hold the same bits).
            const int64_t xs = xchg_floats<M, D>();
            float* xb = p.xbuf + (static_cast<int64_t>(bh) * 2 + (s & 1)) * P * xs;
            const __amdgpu_buffer_rsrc_t xr = xrsrc(xb, static_cast<uint32_t>(P * xs * sizeof(float)));
            {
                const uint32_t mine = static_cast<uint32_t>(pidx * xs) * 4;
#pragma unroll
                for (int db = 0; db < DB; ++db)
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, u[db]), xr,
                                                           mine + ((w * DB + db) * 64 + lane) * 16, 0, XCPOL_SC1);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(aend), xr,
                                                      mine + ((M / 16) * DB * 64 * 4 + w * 64 + lane) * 4, 0,
                                                      XCPOL_SC1);
            }
            // Each wave hands off its own slot rows: they are all that the
            // same wave of the other workgroups reads, so the counters are
            // per (workgroup, wave) and no workgroup barrier is needed.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // this wave's hand-off stores have retired
            int* myflag = p.xflags + ((bh * P + pidx) * G::NWS + w) * XFLAG_STRIDE;
            if (lane == 0) __hip_atomic_store(myflag, s + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            const uint32_t t_off = ((M / 16) * DB * 64 * 4 + w * 64 + lane) * 4;
            if constexpr (!ENC && !LIN1) {
                // Lane j < P - 1 polls the counter of the j-th other workgroup, all
                // in one round trip; then the parts in q order, the workgroup's own
                // from its registers.
                if (!xbroken) {
                    const int j = lane < P - 1 ? lane : 0;
                    const int qj = j < pidx ? j : j + 1;
                    const int* f = p.xflags + ((bh * P + qj) * G::NWS + w) * XFLAG_STRIDE;
                    int n = 0;
                    while (true) {
                        const int v = __hip_atomic_load(const_cast<int*>(f), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        if (__all(lane >= P - 1 || v > s)) break;
                        if (++n >= XSPIN) {
                            xbroken = true;
                            break;
                        }
                    }
                }
                asm volatile("" ::: "memory");  // the reads below stay after the waits
#pragma unroll
                for (int q = 0; q < P; ++q) {
                    if (q == pidx) {
#pragma unroll
                        for (int db = 0; db < DB; ++db)
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[db][e] = fmaf(acc[db][e], aend, u[db][e]);
                        continue;
                    }
                    const uint32_t base = static_cast<uint32_t>(q * xs) * 4;
                    const float tq = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(xr, base + t_off, 0, XCPOL_SC1));
                    f32x4 uq[DB];
#pragma unroll
                    for (int db = 0; db < DB; ++db)
                        uq[db] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, base + ((w * DB + db) * 64 + lane) * 16,
                                                                         0, XCPOL_SC1));
#pragma unroll
                    for (int db = 0; db < DB; ++db)
#pragma unroll
                        for (int e = 0; e < 4; ++e) acc[db][e] = fmaf(acc[db][e], tq, uq[db][e]);
                }
            } else {
                // The encoding and first-linearisation forms hold more
                // registers: every part (its own too) is read back once all
                // are published, R_end = diag(prod_q t_q) Z +
                // sum_q diag(prod_{q' > q} t_q') U_q summed in q order.
#pragma unroll
                for (int q = 0; q < P; ++q)
                    if (q != pidx && !xbroken) xwait<G>(p, bh, P, q, w, s, xbroken);
                asm volatile("" ::: "memory");  // the reads below stay after the waits
                float tq[P];
#pragma unroll
                for (int q = 0; q < P; ++q)
                    tq[q] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                        xr, static_cast<uint32_t>(q * xs) * 4 + ((M / 16) * DB * 64 * 4 + w * 64 + lane) * 4, 0,
                        XCPOL_SC1));
                float sq[P], t_all = 1.f;
#pragma unroll
                for (int q = P - 1; q >= 0; --q) {
                    sq[q] = t_all;
                    t_all *= tq[q];
                }
#pragma unroll
                for (int db = 0; db < DB; ++db)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[db][e] *= t_all;
                // the parts in two batches of q (at most two parts of loads in
                // flight in registers), each added in q order
                constexpr int QB = P < 2 ? P : 2;
#pragma unroll
                for (int q0 = 0; q0 < P; q0 += QB) {
                    f32x4 uq[QB][DB];
#pragma unroll
                    for (int qi = 0; qi < QB; ++qi)
#pragma unroll
                        for (int db = 0; db < DB; ++db)
                            uq[qi][db] = __builtin_bit_cast(
                                f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           xr, static_cast<uint32_t>((q0 + qi) * xs) * 4 + ((w * DB + db) * 64 + lane) * 16,
                                           0, XCPOL_SC1));
#pragma unroll
                    for (int qi = 0; qi < QB; ++qi)
#pragma unroll
                        for (int db = 0; db < DB; ++db)
#pragma unroll
                            for (int e = 0; e < 4; ++e) acc[db][e] = fmaf(sq[q0 + qi], uq[qi][db][e], acc[db][e]);
                }
            }
        } else {
#pragma unroll
            for (int db = 0; db < DB; ++db) acc[db] = u[db];
        }
    }

    if (RAW && grp == 0) {
        float* dst = p.raw + bh * p.raw_stride + static_cast<int64_t>(p.T / C) * M * D +
                     static_cast<int64_t>(slot) * D + 4 * lg;
#pragma unroll
        for (int j = 0; j < DB; ++j) *reinterpret_cast<f32x4*>(dst + 16 * j) = acc[j];
    }
    if (n1 < NC) {
        // hand the unprojected state on to the next chunk range
        if (grp == 0 && pidx == 0) {
            float* dst = p.carry + static_cast<int64_t>(bh) * M * D + static_cast<int64_t>(slot) * D + 4 * lg;
#pragma unroll
            for (int j = 0; j < DB; ++j) *reinterpret_cast<f32x4*>(dst + 16 * j) = acc[j];
        }
        return;
    }
    const float inv = row_inv_norm<DB>(acc);
    if (grp == 0 && pidx == 0 && p.state_out) {
        float* dst = p.state_out + static_cast<int64_t>(bh) * M * D + static_cast<int64_t>(slot) * D + 4 * lg;
#pragma unroll
        for (int j = 0; j < DB; ++j) {
            f32x4 z = acc[j];
#pragma unroll
            for (int r = 0; r < 4; ++r) z[r] *= inv;
            *reinterpret_cast<f32x4*>(dst + 16 * j) = z;
        }
    }
}

}  // namespace mfma
}  // namespace osr
