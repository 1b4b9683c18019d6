// osr_device.h -- device-side helpers shared by the OSR kernels (gfx950).
//
// Element conversion, input loads, wave64 reductions and the kernel parameter
// block.  Nothing here is specific to one kernel.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace osr {

// Kernel parameter block.  Pointers are device pointers; layouts as in
// include/lattice_osr.h ([B,T,H,m] / [B,T,H,d] / [B,T,H] / [B,H,m,d]).
struct Params {
    const void* q;
    const void* k;
    const void* v;
    const void* gamma;
    const void* mu;
    const float* state_in;
    float* state_out;
    void* y;
    float* zbuf;       // chunk-start states [B,H,NC,m,d] (split chunk path only)
    float* raw;        // if set (backward): every chunk-start state before projection, and the
                       // end state, row-major [m][d], at raw + bh * raw_stride + n * m * d
    int64_t raw_stride;
    float* raw_c;      // if set (backward): c and beta of every token and slot, [B*H*NC][m*C] in
    float* raw_b;      // the layout of the gates, and |h|^2 of every token, [B*H*NC][C]
    float* raw_hh;
    float* hrec;       // if set (backward, small chunks, decoding objective): h of every token,
                       // [B*H][T][d] fp32 (the small-chunk token loop only)
    int B, T, H;
    int chunk;         // C
    int gamma_per_slot;
    int mode;          // 0 = decoding objective, 1 = similarity objective, 2 = encoding layer
    int lin1;          // 1: first chunk linearisation (token loop, or the split MFMA schedule)
    int y_bf16;        // 1: y is bf16, 0: y is fp32
    int schedule;      // matrix-core chunk schedule: 0 automatic, 1 split, 2 fused
    int chain_pairs;   // state passing: 0 pairs where they pay, 1 one wave per slot block
    int chain_wgs;     // state passing: 0 split over workgroups where it applies, 1 one workgroup
    int readout_overlap;  // split schedule: 0 read-out overlapped by chunk ranges where it applies, 1 not
    int chain_p;       // workgroups per sequence of the state passing (set by the launch; 1 = not split)
    // State passing with P > 1 workgroups per (b,h) (each takes one sub-block
    // of every chunk): per (b,h), chunk parity and workgroup, that
    // workgroup's part of the chunk-end update and its gate products; and one
    // progress counter per workgroup (128 bytes apart), zeroed before the launch.
    float* xbuf;
    int* xflags;
    // Chunk range of a split-schedule launch: chunks [n_begin, n_end) (n_end = 0:
    // all).  Between ranges the state passing hands the unprojected state on
    // through carry ([B*H][m][d] fp32); only the last range writes state_out.
    int n_begin, n_end;
    float* carry;
    // GeLU post-gate of the layer fused into the y store: y_t <- y_t * GeLU(gate_t)
    // with gate [B,T,H,d] in the inputs' dtype, or null (plain y).
    const void* gate;
};

// ---------------------------------------------------------------- bf16 ----
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round-to-nearest-even float -> bf16 bits (the hardware conversion on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float x) {
    __bf16 h = static_cast<__bf16>(x);
    return __builtin_bit_cast(uint16_t, h);
}

// Element loaders: TIn is float (fp32 inputs) or uint16_t (bf16 bit patterns).
template <typename TIn>
__device__ __forceinline__ float ld(const TIn* p, int64_t i);

template <>
__device__ __forceinline__ float ld<float>(const float* p, int64_t i) {
    return p[i];
}
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

// Four consecutive elements (i must be a multiple of 4).
template <typename TIn>
__device__ __forceinline__ float4 ld4(const TIn* p, int64_t i);

template <>
__device__ __forceinline__ float4 ld4<float>(const float* p, int64_t i) {
    return *reinterpret_cast<const float4*>(p + i);
}
template <>
__device__ __forceinline__ float4 ld4<uint16_t>(const uint16_t* p, int64_t i) {
    const uint2 u = *reinterpret_cast<const uint2*>(p + i);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

// GeLU(x) = x Phi(x), the exact form (Phi through erfc, which keeps its
// relative accuracy in the negative tail where 1 + erf cancels): the layer's
// post-gate on the recurrence's output (section "Experiments", the Lattice
// block).
__device__ __forceinline__ float gelu(float x) { return x * (0.5f * erfcf(-x * 0.70710678118654752f)); }

// Store four consecutive y values as fp32 or bf16.
__device__ __forceinline__ void st_y4(void* y, int64_t i, float4 val, int y_bf16) {
    if (y_bf16) {
        uint2 u;
        u.x = static_cast<uint32_t>(f32_to_bf16_bits(val.x)) |
              (static_cast<uint32_t>(f32_to_bf16_bits(val.y)) << 16);
        u.y = static_cast<uint32_t>(f32_to_bf16_bits(val.z)) |
              (static_cast<uint32_t>(f32_to_bf16_bits(val.w)) << 16);
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(y) + i) = u;
    } else {
        *reinterpret_cast<float4*>(static_cast<float*>(y) + i) = val;
    }
}

__device__ __forceinline__ void st_y1(void* y, int64_t i, float val, int y_bf16) {
    if (y_bf16)
        static_cast<uint16_t*>(y)[i] = f32_to_bf16_bits(val);
    else
        static_cast<float*>(y)[i] = val;
}

// Streaming (non-temporal) 16-byte loads/stores of fp32 state rows.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Hand-offs between the workgroups of one launch (a sequence split over
// several workgroups).  The data goes with the device-coherence bit (sc1):
// such accesses bypass the non-coherent caches (the per-XCD L2 included), so
// readers on any XCD see the data once the writer's stores have retired; no
// write-back or invalidation of the rest of the cache is needed.  Buffer
// instructions keep them ordinary loads and stores for the compiler (issued
// back to back).  A writer's stores retire (s_waitcnt vmcnt(0)) before it
// sets its progress counter with an agent-scope atomic store; a reader polls
// the counter with agent-scope atomic loads, at most XSPIN times.
constexpr int XFLAG_STRIDE = 32;  // ints between progress counters (128 bytes)
constexpr int XSPIN = 1 << 22;    // polls before a wait gives up (never reached when all run)
constexpr int XCPOL_SC1 = 16;     // cache-policy operand: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t xrsrc(float* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ float4 ld_nt4(const float* p) {
    const f32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void st_nt4(float* p, float4 a) {
    f32x4_t v = {a.x, a.y, a.z, a.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4_t*>(p));
}

// -------------------------------------------------------------- float4 ----
__device__ __forceinline__ float4 f4(float a) { return make_float4(a, a, a, a); }
__device__ __forceinline__ float4 operator+(float4 a, float4 b) {
    return make_float4(a.x + b.x, a.y + b.y, a.z + b.z, a.w + b.w);
}
__device__ __forceinline__ float4 operator-(float4 a, float4 b) {
    return make_float4(a.x - b.x, a.y - b.y, a.z - b.z, a.w - b.w);
}
__device__ __forceinline__ float4 operator*(float s, float4 a) {
    return make_float4(s * a.x, s * a.y, s * a.z, s * a.w);
}
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 c) {
    return make_float4(fmaf(s, a.x, c.x), fmaf(s, a.y, c.y), fmaf(s, a.z, c.z), fmaf(s, a.w, c.w));
}
__device__ __forceinline__ float dot4(float4 a, float4 b) {
    return fmaf(a.x, b.x, fmaf(a.y, b.y, fmaf(a.z, b.z, a.w * b.w)));
}

// ---------------------------------------------------------- reductions ----
// Cross-lane moves on the vector ALU: DPP inside 16-lane rows, and the gfx950
// row swaps across rows (no LDS round trip, unlike a shuffle through
// ds_bpermute).
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int DPP_QUAD_1032 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;   // lane i <- lane 15 - i of its row
constexpr int DPP_HALF_MIRROR = 0x141;  // lane i <- lane 7 - i of its half row
constexpr int DPP_ROW_ROR = 0x120;      // + n: lane i <- lane (i + n) % 16 of its row

// Value of the same lane column in the even and in the odd row of the lane's
// row pair (rows 0/1, 2/3), and in the lower and upper half of the wave.
__device__ __forceinline__ void row_pair_values(float x, float& even, float& odd) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    even = __uint_as_float(r[0]);
    odd = __uint_as_float(r[1]);
}
__device__ __forceinline__ void wave_half_values(float x, float& lo, float& hi) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    lo = __uint_as_float(r[0]);
    hi = __uint_as_float(r[1]);
}

// Sum over groups of G consecutive lanes of a wave64 (G a power of two <= 64);
// every lane of the group receives the sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(G >= 1 && G <= 64 && (G & (G - 1)) == 0, "power of two");
    if constexpr (G >= 2) x += dpp_mov<DPP_QUAD_1032>(x);
    if constexpr (G >= 4) x += dpp_mov<DPP_QUAD_2301>(x);
    if constexpr (G >= 8) x += dpp_mov<DPP_HALF_MIRROR>(x);
    if constexpr (G >= 16) x += dpp_mov<DPP_ROW_MIRROR>(x);
    if constexpr (G >= 32) {
        float e, o;
        row_pair_values(x, e, o);
        x = e + o;
    }
    if constexpr (G >= 64) {
        float lo, hi;
        wave_half_values(x, lo, hi);
        x = lo + hi;
    }
    return x;
}

// Sum over each row of 16 lanes (lanes 16r .. 16r+15) with DPP row
// rotations; every lane of the row receives the sum.
__device__ __forceinline__ float row16_sum(float x) {
    x += dpp_mov<DPP_ROW_ROR + 8>(x);
    x += dpp_mov<DPP_ROW_ROR + 4>(x);
    x += dpp_mov<DPP_ROW_ROR + 2>(x);
    x += dpp_mov<DPP_ROW_ROR + 1>(x);
    return x;
}

// Sum over lanes that share (lane % S), S a power of two < 64.  Every lane
// receives the sum of its class.
template <int S>
__device__ __forceinline__ float strided_sum(float x) {
    static_assert(S >= 1 && S < 64 && (S & (S - 1)) == 0, "power of two below 64");
    if constexpr (S <= 8) x += dpp_mov<DPP_ROW_ROR + 8>(x);
    if constexpr (S <= 4) x += dpp_mov<DPP_ROW_ROR + 4>(x);
    if constexpr (S <= 2) x += dpp_mov<DPP_ROW_ROR + 2>(x);
    if constexpr (S <= 1) x += dpp_mov<DPP_ROW_ROR + 1>(x);
    if constexpr (S <= 16) {
        float e, o;
        row_pair_values(x, e, o);
        x = e + o;
    }
    float lo, hi;
    wave_half_values(x, lo, hi);
    return lo + hi;
}

}  // namespace osr
