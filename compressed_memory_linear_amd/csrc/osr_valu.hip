// osr_valu.hip -- VALU (fp32) OSR kernels for gfx950: the fused single-token
// decode step and the token-by-token forward (exact recurrence at C = 1, the
// chunk-linearised recurrence at C > 1).
//
// Method: "Lattice: Learning to Efficiently Compress the Memory" (arXiv
// 2504.05646).  Per token, with Z the unit-projected chunk-start state
// (section "Stabilizing Memory Updates via Normalization") and S the running
// state, both m x d with row i = slot i:
//   h   = sum_i k_i z_i - v  (decoding objective), -v (similarity) or v
//         (encoding layer, subsection "Encoding layer")
//   c_i = z_i . h,  a_i = gamma_i k_i (gamma_i (c_i - k_i) for the encoding
//         layer: its per-slot error z_i . v - k_i),  w_i = max(|h|^2 - c_i^2, 0)
//   beta_i = (mu^2 + a_i^2 w_i)^(-1/2)            (eq. normalized_recurrence
//                                                  with the forget gate)
//   s_i <- beta_i (mu + a_i c_i) s_i - beta_i a_i h   (eq. recurrence_detailed;
//                                                  eq. recurrence_linear2 when
//                                                  C > 1)
//   or, with the first chunk linearisation (eq. recurrence_linear1),
//   s_i <- beta_i mu s_i + beta_i a_i c_i z_i - beta_i a_i h
//   y   = sum_i q_i s_i                           (memory read-out)
// With C = 1, Z = S and the step is the exact projected orthogonal update.
//
// Thread layout and reductions: osr_valu.h.
#include "osr_launch.h"
#include "osr_valu.h"

namespace osr {

// One token: update the running state s from the chunk-start state z and
// return the read-out for this thread's 4 columns (valid in every thread).
// red_h and red_y must be distinct buffers, and red_y must differ from the
// red_y of the previous call (callers alternate it by token parity): that way
// one barrier per reduction orders every write after the last read of the
// same buffer.
template <class L, int D>
__device__ __forceinline__ float4 osr_token(const float4 (&z)[L::RPT], float4 (&s)[L::RPT],
                                            const TokenIn<L::RPT>& in, int mode, int lin1, float* red_h,
                                            float* red_y, int lane, int wave, int cg) {
    float4 h;
    if (mode == 0) {
        float4 hp = f4(0.f);
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) hp = fma4(in.k[i], z[i], hp);
        h = col_sum<L, D>(hp, red_h, lane, wave, cg) - in.v;
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
    const float hh = cc[L::RPT];
    const float mu = in.mu;
    float4 yp = f4(0.f);
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) {
        const float a = in.g[i] * (mode == 2 ? cc[i] - in.k[i] : in.k[i]);
        const float w = fmaxf(fmaf(-cc[i], cc[i], hh), 0.f);
        const float beta = rsqrtf(fmaf(mu, mu, a * a * w));
        const float kap = -beta * a;
        if (lin1) {
            // mu beta on the running slot, the projection term on z
            s[i] = fma4(beta * mu, s[i], fma4(beta * a * cc[i], z[i], kap * h));
        } else {
            const float gate = beta * fmaf(a, cc[i], mu);
            s[i] = fma4(gate, s[i], kap * h);
        }
        yp = fma4(in.q[i], s[i], yp);
    }
    return col_sum<L, D>(yp, red_y, lane, wave, cg);
}

// ------------------------------------------------------------------ decode --
template <int M, int D, int NT, typename TIn>
__global__ __launch_bounds__(NT) void osr_decode_kernel(Params p) {
    using L = ValuLayout<M, D, NT>;
    __shared__ float red[2][L::NW * D];
    const int bh = blockIdx.x;  // T == 1: token index b*H + h
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % L::TPR, rg = tid / L::TPR;

    const float* sin = p.state_in + static_cast<int64_t>(bh) * M * D;
    float4 s[L::RPT];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i)
        s[i] = ld_nt4(sin + (rg + L::RG * i) * D + cg * 4);
    TokenIn<L::RPT> in;
    load_token<L, M, D, TIn>(in, p, bh, rg, cg);

    project_rows<L>(s);
    float4 z[L::RPT];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i) z[i] = s[i];
    const float4 y = osr_token<L, D>(z, s, in, p.mode, 0, red[0], red[1], lane, wave, cg);
    if (rg == 0) st_y4(p.y, static_cast<int64_t>(bh) * D + cg * 4, y, p.y_bf16);

    project_rows<L>(s);
    float* sout = p.state_out + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i)
        st_nt4(sout + (rg + L::RG * i) * D + cg * 4, s[i]);
}

// -------------------------------------------------------------- token loop --
template <int M, int D, int NT, typename TIn>
__global__ __launch_bounds__(NT) void osr_tokenloop_kernel(Params p) {
    using L = ValuLayout<M, D, NT>;
    __shared__ float red[3][L::NW * D];
    const int bh = blockIdx.x;
    const int b = bh / p.H, hd = bh % p.H;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int cg = tid % L::TPR, rg = tid / L::TPR;
    const int T = p.T, C = p.chunk;

    const float* sin = p.state_in + static_cast<int64_t>(bh) * M * D;
    float4 s[L::RPT], z[L::RPT];
#pragma unroll
    for (int i = 0; i < L::RPT; ++i)
        s[i] = *reinterpret_cast<const float4*>(sin + (rg + L::RG * i) * D + cg * 4);

    auto bth_of = [&](int t) { return (static_cast<int64_t>(b) * T + t) * p.H + hd; };
    TokenIn<L::RPT> cur, nxt;
    load_token<L, M, D, TIn>(cur, p, bth_of(0), rg, cg);

    for (int t0 = 0; t0 < T; t0 += C) {
        project_rows<L>(s);
#pragma unroll
        for (int i = 0; i < L::RPT; ++i) z[i] = s[i];
        for (int t = t0; t < t0 + C; ++t) {
            if (t + 1 < T) load_token<L, M, D, TIn>(nxt, p, bth_of(t + 1), rg, cg);
            const float4 y = osr_token<L, D>(z, s, cur, p.mode, p.lin1, red[2], red[t & 1], lane, wave, cg);
            if (rg == 0) st_y4(p.y, bth_of(t) * D + cg * 4, y, p.y_bf16);
            cur = nxt;
        }
    }
    project_rows<L>(s);
    float* sout = p.state_out + static_cast<int64_t>(bh) * M * D;
#pragma unroll
    for (int i = 0; i < L::RPT; ++i)
        *reinterpret_cast<float4*>(sout + (rg + L::RG * i) * D + cg * 4) = s[i];
}

// ----------------------------------------------------------------- launch --
template <int M, int D>
static int launch_valu_md(bool decode, const Params& p, bool in_bf16, hipStream_t st) {
    constexpr int TPR = D / 4;
    // Decode: up to 8 waves per state (fewer rows per thread: ~100 VGPRs, 4 waves per SIMD), which
    // shortens each workgroup's arithmetic between its state load and store; measured 9% faster
    // than 4 waves at m = d = 128.
    constexpr int NT_DEC = (M * TPR < 512) ? M * TPR : 512;
    constexpr int NT_TOK = (M * TPR < 512) ? M * TPR : 512;
    const dim3 grid(static_cast<unsigned>(p.B) * static_cast<unsigned>(p.H));
    if (decode) {
        if (in_bf16)
            hipLaunchKernelGGL((osr_decode_kernel<M, D, NT_DEC, uint16_t>), grid, dim3(NT_DEC), 0, st, p);
        else
            hipLaunchKernelGGL((osr_decode_kernel<M, D, NT_DEC, float>), grid, dim3(NT_DEC), 0, st, p);
    } else {
        if (in_bf16)
            hipLaunchKernelGGL((osr_tokenloop_kernel<M, D, NT_TOK, uint16_t>), grid, dim3(NT_TOK), 0, st, p);
        else
            hipLaunchKernelGGL((osr_tokenloop_kernel<M, D, NT_TOK, float>), grid, dim3(NT_TOK), 0, st, p);
    }
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

template <int M>
static int launch_valu_m(bool decode, int d, const Params& p, bool in_bf16, hipStream_t st) {
    switch (d) {
        case 16: return launch_valu_md<M, 16>(decode, p, in_bf16, st);
        case 32: return launch_valu_md<M, 32>(decode, p, in_bf16, st);
        case 64: return launch_valu_md<M, 64>(decode, p, in_bf16, st);
        case 128: return launch_valu_md<M, 128>(decode, p, in_bf16, st);
        default: return -3;
    }
}

int launch_valu(bool decode, int m, int d, const Params& p, bool in_bf16, hipStream_t st) {
    switch (m) {
        case 16: return launch_valu_m<16>(decode, d, p, in_bf16, st);
        case 32: return launch_valu_m<32>(decode, d, p, in_bf16, st);
        case 64: return launch_valu_m<64>(decode, d, p, in_bf16, st);
        case 128: return launch_valu_m<128>(decode, d, p, in_bf16, st);
        default: return -3;
    }
}

}  // namespace osr
