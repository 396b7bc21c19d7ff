// Device-side helpers shared by the gfx950 kernels of the MoE glue path.
// Wave64 throughout; 16-byte (dwordx4) global accesses per lane.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
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

}  // namespace moe
