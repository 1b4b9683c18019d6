// osr_glue.hip -- the layer glue around the recurrence, as two streaming kernels.
//
// "Lattice: Learning to Efficiently Compress the Memory" (arXiv 2504.05646),
// section "Experiments", paragraph on the Lattice block, and the
// experiment-details appendix: q and k each pass through a short causal 1-D
// convolution of width 4 (one filter per channel), the writing intensity is
// gamma = sigmoid(W_gamma x), and the recurrence's output passes through a
// GeLU post-gate.  The projections themselves (W_gamma x, the gate branch) are
// the caller's GEMMs; these kernels do everything between them and the
// recurrence in one pass over HBM each:
//
//   pre:  q = conv4(xq), k = conv4(xk), gamma = sigmoid(logit), and the last
//         three raw q/k rows as the history of the next call;
//   post: out = y * GeLU(g), GeLU(x) = x Phi(x) = x erfc(-x / sqrt 2) / 2.
//
// Both are bound by HBM bandwidth: every input element is read once (plus a
// three-token halo per 64-token tile of the convolution, which the L2 serves)
// and every output element written once, in 16-byte pieces.  Arithmetic is
// fp32; bf16 inputs are widened exactly and outputs rounded to nearest even.
#include <hip/hip_runtime.h>

#include "osr_launch.h"

namespace osr {
namespace {

constexpr int kTaps = 4;        // width of the short convolution
constexpr int kVec = 8;         // channels per thread (16 bytes of bf16)
constexpr int kTile = 64;       // tokens per thread in the convolution
constexpr int kPreThreads = 64; // one wave per workgroup
constexpr int kAhead = 8;       // rows loaded ahead of their use

// Eight consecutive elements as fp32, from fp32 or bf16 storage (16-byte aligned).
__device__ __forceinline__ void load8(const float* p, int64_t i, float (&x)[kVec]) {
    const float4 a = *reinterpret_cast<const float4*>(p + i);
    const float4 b = *reinterpret_cast<const float4*>(p + i + 4);
    x[0] = a.x, x[1] = a.y, x[2] = a.z, x[3] = a.w, x[4] = b.x, x[5] = b.y, x[6] = b.z, x[7] = b.w;
}
__device__ __forceinline__ void load8(const uint16_t* p, int64_t i, float (&x)[kVec]) {
    const uint4 u = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void store8(float* p, int64_t i, const float (&x)[kVec]) {
    *reinterpret_cast<float4*>(p + i) = make_float4(x[0], x[1], x[2], x[3]);
    *reinterpret_cast<float4*>(p + i + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(uint16_t* p, int64_t i, const float (&x)[kVec]) {
    uint32_t w[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        w[j] = static_cast<uint32_t>(f32_to_bf16_bits(x[2 * j])) |
               (static_cast<uint32_t>(f32_to_bf16_bits(x[2 * j + 1])) << 16);
    *reinterpret_cast<uint4*>(p + i) = make_uint4(w[0], w[1], w[2], w[3]);
}
// Eight elements as stored, so a batch of rows can be in flight at once in few registers.
template <typename T>
struct Raw8;
template <>
struct Raw8<uint16_t> {
    uint4 u;
};
template <>
struct Raw8<float> {
    float4 a, b;
};
__device__ __forceinline__ void load_raw(const uint16_t* p, int64_t i, Raw8<uint16_t>& r) {
    r.u = *reinterpret_cast<const uint4*>(p + i);
}
__device__ __forceinline__ void load_raw(const float* p, int64_t i, Raw8<float>& r) {
    r.a = *reinterpret_cast<const float4*>(p + i);
    r.b = *reinterpret_cast<const float4*>(p + i + 4);
}
__device__ __forceinline__ void widen(const Raw8<uint16_t>& r, float (&x)[kVec]) {
    const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        x[2 * j] = __uint_as_float(w[j] << 16);
        x[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}
__device__ __forceinline__ void widen(const Raw8<float>& r, float (&x)[kVec]) {
    x[0] = r.a.x, x[1] = r.a.y, x[2] = r.a.z, x[3] = r.a.w, x[4] = r.b.x, x[5] = r.b.y, x[6] = r.b.z, x[7] = r.b.w;
}
__device__ __forceinline__ float load1(const float* p, int64_t i) { return p[i]; }
__device__ __forceinline__ float load1(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }
__device__ __forceinline__ void store1(float* p, int64_t i, float x) { p[i] = x; }
__device__ __forceinline__ void store1(uint16_t* p, int64_t i, float x) { p[i] = f32_to_bf16_bits(x); }

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + expf(-x)); }

// Work unit u of a token tile: u < 2 nc is a group of 8 q (u < nc) or k
// channels; the rest are groups of up to 8 gamma logits.
template <typename TIn>
__global__ __launch_bounds__(kPreThreads) void osr_glue_pre_kernel(GlueParams p) {
    const int nc = p.N / kVec;
    const int ng = (p.G + kVec - 1) / kVec;
    const int ub = (2 * nc + ng + kPreThreads - 1) / kPreThreads;  // workgroups per token tile
    const int u = static_cast<int>(blockIdx.x % ub) * kPreThreads + threadIdx.x;
    if (u >= 2 * nc + ng) return;
    const int tiles = (p.T + kTile - 1) / kTile;
    const int tile = static_cast<int>(blockIdx.x / ub);  // consecutive workgroups share a tile
    const int b = tile / tiles;
    const int t0 = (tile % tiles) * kTile;
    const int t1 = min(t0 + kTile, p.T);

    if (u >= 2 * nc) {
        // gamma = sigmoid(logit): rows of G values, vector pieces where G allows
        const TIn* lg = static_cast<const TIn*>(p.glogit);
        TIn* gm = static_cast<TIn*>(p.gamma);
        const int e0 = (u - 2 * nc) * kVec;
        auto grow = [&](int t) { return (static_cast<int64_t>(b) * p.T + t) * p.G + e0; };
        if (p.gvec) {
            auto emit = [&](const Raw8<TIn>& r, int t) {
                float v[kVec];
                widen(r, v);
#pragma unroll
                for (int j = 0; j < kVec; ++j) v[j] = sigmoid(v[j]);
                store8(gm, grow(t), v);
            };
            Raw8<TIn> ring[kAhead];
#pragma unroll
            for (int i = 0; i < kAhead; ++i) load_raw(lg, grow(min(t0 + i, t1 - 1)), ring[i]);
            const int tfull = t0 + (t1 - t0) / kAhead * kAhead;
            for (int tb = t0; tb < tfull; tb += kAhead) {
#pragma unroll
                for (int i = 0; i < kAhead; ++i) {
                    const Raw8<TIn> r = ring[i];
                    load_raw(lg, grow(min(tb + i + kAhead, t1 - 1)), ring[i]);
                    emit(r, tb + i);
                }
            }
#pragma unroll
            for (int i = 0; i < kAhead - 1; ++i)
                if (tfull + i < t1) emit(ring[i], tfull + i);
        } else {
            for (int t = t0; t < t1; ++t)
                for (int e = e0; e < min(e0 + kVec, p.G); ++e) store1(gm, grow(t) - e0 + e, sigmoid(load1(lg, grow(t) - e0 + e)));
        }
        return;
    }

    const bool is_k = u >= nc;
    const int c0 = (is_k ? u - nc : u) * kVec;  // first channel of this thread
    const TIn* x = static_cast<const TIn*>(is_k ? p.xk : p.xq);
    const TIn* hin = static_cast<const TIn*>(is_k ? p.hk_in : p.hq_in);
    const float* w = is_k ? p.wk : p.wq;
    const float* bias = is_k ? p.bk : p.bq;
    TIn* out = static_cast<TIn*>(is_k ? p.k : p.q);
    TIn* hout = static_cast<TIn*>(is_k ? p.hk_out : p.hq_out);

    float wt[kTaps][kVec], bv[kVec];
#pragma unroll
    for (int j = 0; j < kVec; ++j) {
        const float4 f = *reinterpret_cast<const float4*>(w + static_cast<int64_t>(c0 + j) * kTaps);
        wt[0][j] = f.x, wt[1][j] = f.y, wt[2][j] = f.z, wt[3][j] = f.w;
        bv[j] = bias ? bias[c0 + j] : 0.0f;
    }
    // Row s of the sequence extended by the history (s in [-3, T)).
    auto fetch = [&](int s, float (&r)[kVec]) {
        if (s >= 0) {
            load8(x, (static_cast<int64_t>(b) * p.T + s) * p.N + c0, r);
        } else if (hin) {
            load8(hin, (static_cast<int64_t>(b) * (kTaps - 1) + (s + kTaps - 1)) * p.N + c0, r);
        } else {
#pragma unroll
            for (int j = 0; j < kVec; ++j) r[j] = 0.0f;
        }
    };
    float win[kTaps - 1][kVec];  // rows t-3, t-2, t-1
    fetch(t0 - 3, win[0]);
    fetch(t0 - 2, win[1]);
    fetch(t0 - 1, win[2]);
    // Rows are loaded kAhead tokens before their use, each load issued ahead of
    // the store of the row before it: a wave's counter of outstanding memory
    // operations drains in issue order, so a load waited on right after a
    // store would wait for that store's completion too.  The loads are
    // unconditional (past the tile's end they repeat its last row) and the
    // main loop takes whole groups of rows, so that no branch forces an early
    // wait.  104 -> 92 us for B8 H16 T4096 m64 (bf16) at 4 rows ahead and
    // 32-token tiles; 8 rows ahead and 64-token tiles (half the halo re-reads)
    // 94-97 -> 91-92 us; 128-token tiles 104 us (too few waves for the chip).
    auto xrow = [&](int t) { return (static_cast<int64_t>(b) * p.T + t) * p.N + c0; };
    auto emit = [&](const Raw8<TIn>& r, int t) {
        float cur[kVec], o[kVec];
        widen(r, cur);
#pragma unroll
        for (int j = 0; j < kVec; ++j) {
            float a = bv[j];
            a = fmaf(wt[0][j], win[0][j], a);
            a = fmaf(wt[1][j], win[1][j], a);
            a = fmaf(wt[2][j], win[2][j], a);
            a = fmaf(wt[3][j], cur[j], a);
            o[j] = a;
            win[0][j] = win[1][j];
            win[1][j] = win[2][j];
            win[2][j] = cur[j];
        }
        store8(out, xrow(t), o);
    };
    Raw8<TIn> ring[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) load_raw(x, xrow(min(t0 + i, t1 - 1)), ring[i]);
    const int tfull = t0 + (t1 - t0) / kAhead * kAhead;  // whole groups of kAhead rows
    for (int tb = t0; tb < tfull; tb += kAhead) {
#pragma unroll
        for (int i = 0; i < kAhead; ++i) {
            const Raw8<TIn> r = ring[i];
            load_raw(x, xrow(min(tb + i + kAhead, t1 - 1)), ring[i]);
            emit(r, tb + i);
        }
    }
    // the last (up to 3) rows of a ragged tile are already in the ring
#pragma unroll
    for (int i = 0; i < kAhead - 1; ++i)
        if (tfull + i < t1) emit(ring[i], tfull + i);
    // the last tile hands the final three raw rows on as the next call's history
    if (hout && t1 == p.T) {
#pragma unroll
        for (int r = 0; r < kTaps - 1; ++r) {
            float v[kVec];
            fetch(p.T - (kTaps - 1) + r, v);
            store8(hout, (static_cast<int64_t>(b) * (kTaps - 1) + r) * p.N + c0, v);
        }
    }
}

// out = y * GeLU(g) over n elements, n a multiple of 8, grid-stride; each pass
// issues the loads of kPost pieces of 8 (one stride apart) before using them.
constexpr int kPost = 4;
template <typename TY, typename TG>
__global__ __launch_bounds__(256) void osr_glue_post_kernel(const TY* y, const TG* __restrict__ g, TY* out,
                                                            int64_t n) {
    // out may be y itself: each element is read and written by one thread, in that order
    const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x * kVec;
    for (int64_t i0 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * kVec; i0 < n;
         i0 += kPost * stride) {
        Raw8<TY> ry[kPost];
        Raw8<TG> rg[kPost];
        // unconditional loads (a piece past the end reads the thread's own first
        // piece again, which it writes only after every load): a load under a
        // branch is waited for where the branch joins
#pragma unroll
        for (int k = 0; k < kPost; ++k) {
            const int64_t ik = i0 + k * stride < n ? i0 + k * stride : i0;
            load_raw(y, ik, ry[k]);
            load_raw(g, ik, rg[k]);
        }
#pragma unroll
        for (int k = 0; k < kPost; ++k) {
            if (i0 + k * stride < n) {
                float yv[kVec], gv[kVec];
                widen(ry[k], yv);
                widen(rg[k], gv);
#pragma unroll
                for (int j = 0; j < kVec; ++j) yv[j] *= gelu(gv[j]);
                store8(out, i0 + k * stride, yv);
            }
        }
    }
}

}  // namespace

int launch_glue_pre(const GlueParams& p, bool in_bf16, hipStream_t st) {
    if (p.N % kVec != 0 || p.B <= 0 || p.T <= 0 || p.G <= 0) return -3;
    const int64_t units = 2 * (p.N / kVec) + (p.G + kVec - 1) / kVec;
    const int64_t blocks = (units + kPreThreads - 1) / kPreThreads * p.B * ((p.T + kTile - 1) / kTile);
    if (blocks > 2147483647) return -3;
    const dim3 grid(static_cast<unsigned>(blocks));
    if (in_bf16)
        hipLaunchKernelGGL(osr_glue_pre_kernel<uint16_t>, grid, dim3(kPreThreads), 0, st, p);
    else
        hipLaunchKernelGGL(osr_glue_pre_kernel<float>, grid, dim3(kPreThreads), 0, st, p);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

int launch_glue_post(const void* y, bool y_bf16, const void* g, bool g_bf16, void* out, int64_t n, hipStream_t st) {
    if (n % kVec != 0) return -3;
    // enough workgroups for every CU several times over, then grid-stride
    const int64_t want = (n / kVec / kPost + 255) / 256;
    const unsigned blocks = static_cast<unsigned>(want < 8192 ? (want > 0 ? want : 1) : 8192);
    if (y_bf16 && g_bf16)
        hipLaunchKernelGGL((osr_glue_post_kernel<uint16_t, uint16_t>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint16_t*>(y), static_cast<const uint16_t*>(g),
                           static_cast<uint16_t*>(out), n);
    else if (y_bf16)
        hipLaunchKernelGGL((osr_glue_post_kernel<uint16_t, float>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const uint16_t*>(y), static_cast<const float*>(g), static_cast<uint16_t*>(out),
                           n);
    else if (g_bf16)
        hipLaunchKernelGGL((osr_glue_post_kernel<float, uint16_t>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const float*>(y), static_cast<const uint16_t*>(g), static_cast<float*>(out), n);
    else
        hipLaunchKernelGGL((osr_glue_post_kernel<float, float>), dim3(blocks), dim3(256), 0, st,
                           static_cast<const float*>(y), static_cast<const float*>(g), static_cast<float*>(out), n);
    return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // namespace osr
