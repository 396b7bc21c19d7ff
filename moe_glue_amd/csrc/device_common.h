// Device-side helpers shared by the gfx950 kernels of the MoE glue path.
// Wave64 throughout; 16-byte (dwordx4) global accesses per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ------------------------------------------------------------------ bf16
// A 16-byte vector holds 8 bf16 values: word w carries element 2w in its low
// half and element 2w+1 in its high half (little-endian memory order).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// Two fp32 -> bf16 conversions, round to nearest even, in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    bf16x2 b = __builtin_convertvector(v, bf16x2);
    return __builtin_bit_cast(uint32_t, b);
}

__device__ __forceinline__ void unpack8(const u32x4& v, float (&f)[8]) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        f[2 * w] = bf16_lo(v[w]);
        f[2 * w + 1] = bf16_hi(v[w]);
    }
}

__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
    u32x4 v;
#pragma unroll
    for (int w = 0; w < 4; ++w) v[w] = pack_bf16x2(f[2 * w], f[2 * w + 1]);
    return v;
}

// -------------------------------------------------------- global memory
// Streaming accesses: data touched once, so mark them non-temporal.
__device__ __forceinline__ u32x4 load_stream(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_stream(u32x4* p, const u32x4& v) { __builtin_nontemporal_store(v, p); }

// An 8-byte store of item i with the sc1 (system scope) cache bit beside the
// non-temporal one, for the 8-byte lanes of combine and SwiGLU on large
// batches, where it measured faster than nt alone.  No plain global store
// carries sc1, so it is a raw buffer store through a resource covering the
// wave's items [i0, min(n, i0 + 64)), i0 <= i < n: stride 0, so num_records
// counts bytes, and word 3 sets the 32-bit data format, without which a gfx9
// buffer access is out of range.
constexpr int kRawBufferWord3 = 0x00020000;
constexpr int kCacheNt = 2;
constexpr int kCacheSc1 = 16;
__device__ __forceinline__ void store_stream_sc1(u32x2* out, uint32_t i0, uint32_t i, uint32_t n, const u32x2& v) {
    const int bytes = (int)(min(n - i0, (uint32_t)kWave) * (uint32_t)sizeof(u32x2));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(out + i0, 0, bytes, kRawBufferWord3);
    __builtin_amdgcn_raw_buffer_store_b64(v, rs, (int)((i - i0) * sizeof(u32x2)), 0, kCacheNt | kCacheSc1);
}

// ------------------------------------------------------- integer division
// Unsigned division by a runtime constant d >= 1 for n < 2^31, as one
// multiply-high, an add and a shift (the round-up method of Granlund and
// Montgomery, "Division by Invariant Integers using Multiplication", 1994).
struct FastDiv {
    uint32_t d;
    uint32_t mul;
    uint32_t shift;
};

__host__ inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.shift = s;
    // mul = floor(2^32 * (2^s - d) / d) + 1
    f.mul = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
    return f;
}

__host__ __device__ __forceinline__ uint32_t fastdiv(uint32_t n, const FastDiv& f) {
    uint32_t hi = (uint32_t)(((uint64_t)n * f.mul) >> 32);  // v_mul_hi_u32
    return (hi + n) >> f.shift;  // hi <= n < 2^31, so the sum cannot wrap
}

__device__ __forceinline__ uint32_t uniform(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// ------------------------------------------------------ lane-group reductions
// Reductions over each aligned group of G lanes (G a power of two <= 64),
// result in every lane of the group, without the LDS crossbar: DPP quad
// permutations for lane distance 1 and 2, DPP half-row / row mirrors to join
// quads into 8 and 16 lanes, and the gfx950 permlane16/permlane32 swaps to
// join rows into 32 and 64 lanes.  All are VALU operations.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}

constexpr int kQuadXor1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

enum class Op { Max, Min, FAdd };  // unsigned max / min, fp32 add (on the bits)

template <Op OP>
__device__ __forceinline__ uint32_t apply(uint32_t a, uint32_t b) {
    if constexpr (OP == Op::Max) return a > b ? a : b;
    if constexpr (OP == Op::Min) return a < b ? a : b;
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
}

template <int G, Op OP>
__device__ __forceinline__ uint32_t group_reduce(uint32_t v) {
    if constexpr (G > 1) v = apply<OP>(v, dpp<kQuadXor1>(v));
    if constexpr (G > 2) v = apply<OP>(v, dpp<kQuadXor2>(v));
    if constexpr (G > 4) v = apply<OP>(v, dpp<kRowHalfMirror>(v));
    if constexpr (G > 8) v = apply<OP>(v, dpp<kRowMirror>(v));
    if constexpr (G > 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = apply<OP>(p[0], p[1]);
    }
    if constexpr (G > 32) {
        const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        v = apply<OP>(p[0], p[1]);
    }
    return v;
}

// Inclusive prefix sum over the 64 lanes of a wave (every lane active):
// Hillis-Steele shifts of 1, 2, 4 and 8 lanes inside each 16-lane row by DPP
// row_shr (lanes shifted in from outside the row read 0), then each row adds
// the totals of the rows below it, read with v_readlane.
__device__ __forceinline__ int wave_inclusive_sum(int v) {
    v += (int)dpp<0x111>((uint32_t)v);  // row_shr:1
    v += (int)dpp<0x112>((uint32_t)v);  // row_shr:2
    v += (int)dpp<0x114>((uint32_t)v);  // row_shr:4
    v += (int)dpp<0x118>((uint32_t)v);  // row_shr:8
    const int row = (int)(threadIdx.x % kWave) >> 4;
    const int r0 = __builtin_amdgcn_readlane(v, 15);
    const int r1 = __builtin_amdgcn_readlane(v, 31);
    const int r2 = __builtin_amdgcn_readlane(v, 47);
    return v + (row >= 1 ? r0 : 0) + (row >= 2 ? r1 : 0) + (row >= 3 ? r2 : 0);
}

}  // namespace moe
