// OCP E4M3 quantisation of 16-byte bf16 vectors, shared by the quantising
// expand (quant.hip) and the route's place step when it copies the rows
// itself (route.hip).  A scale group of `group` columns is group/8
// consecutive lanes; its absolute maximum is a max over those lanes of the
// fp32 bit patterns of |x| (order-preserving for non-negative values).  Then
// scale = amax/448 and inv = 448/amax (IEEE fp32 divisions; 0 for an all-zero
// group; below amax = 2^-64 x and amax are first scaled by 2^64), the products
// x*inv are clamped to +-448 and converted two at a time by v_cvt_pk_fp8_f32
// (E4M3, nearest-even; the clamp makes it saturating).
#pragma once

#include "device_common.h"

namespace moe {

__device__ __forceinline__ float clamp448(float v) { return fminf(fmaxf(v, -448.0f), 448.0f); }

// Largest |f[e]| of the lane's 8 values, as fp32 bits.
__device__ __forceinline__ uint32_t abs_max_bits8(const float (&f)[8]) {
    uint32_t m = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const uint32_t b = __builtin_bit_cast(uint32_t, f[e]) & 0x7FFFFFFFu;
        m = b > m ? b : m;
    }
    return m;
}

// The group maximum over gl = group/8 consecutive lanes (a power of two <= 64;
// wave-uniform), by DPP/permlane reductions.
__device__ __forceinline__ uint32_t group_abs_max(uint32_t m, int gl) {
    switch (gl) {
        case 1: return m;
        case 2: return group_reduce<2, Op::Max>(m);
        case 4: return group_reduce<4, Op::Max>(m);
        case 8: return group_reduce<8, Op::Max>(m);
        case 16: return group_reduce<16, Op::Max>(m);
        case 32: return group_reduce<32, Op::Max>(m);
        default: return group_reduce<64, Op::Max>(m);
    }
}

__device__ __forceinline__ float e4m3_scale(float amax) { return amax / 448.0f; }
// The inverse scale and the product x * inv are fp32 roundings taken without
// fp32's exponent limits: below amax = 2^-64 (bf16 subnormals and the lowest
// normals, where 448/amax overflows) x and amax are first multiplied by
// pre = 2^64, exactly; elsewhere pre = 1.  The decision is made on amax's bits.
__device__ __forceinline__ float e4m3_prescale(uint32_t amax_bits) {
    return amax_bits < 0x1F800000u ? 0x1p64f : 1.0f;  // 0x1F800000 = 2^-64
}
__device__ __forceinline__ float e4m3_inverse_scale(float amax, float pre) {
    return amax > 0.0f ? 448.0f / (amax * pre) : 0.0f;
}

// OCP microscaling (MX) block scale from the fp32 bits of the block's |x|
// maximum, a bf16 value widened to fp32: e = max(floor(log2 amax) - 8, -127)
// (8 is the exponent of E4M3's largest normal), -127 for a zero or
// subnormal maximum; floor(log2 amax) of a normal amax is its exponent field
// minus 127.  The E8M0 byte is e + 127, and 2^-e -- built from its bits,
// 127 - e in [8, 254] for every finite maximum -- is a normal fp32, so
// x * 2^-e is exact.
__device__ __forceinline__ int mx_scale_exponent(uint32_t amax_bits) {
    const int ef = (int)(amax_bits >> 23);
    return ef == 0 ? -127 : max(ef - 127 - 8, -127);
}
__device__ __forceinline__ float mx_inverse_scale(int e) { return __builtin_bit_cast(float, (uint32_t)(127 - e) << 23); }

// A block's scale in either format: fp32 amax/448 (scale) or MX (byte), and
// the factor the codes are taken of.
struct BlockScale {
    float pre;  // x is multiplied by pre, then by inv (pre = 1 for MX)
    float inv;
    float scale;
    uint8_t byte;
};
__device__ __forceinline__ BlockScale block_scale(uint32_t amax_bits, bool mx) {
    BlockScale b;
    if (mx) {
        const int e = mx_scale_exponent(amax_bits);
        b.pre = 1.0f;
        b.inv = mx_inverse_scale(e);
        b.scale = 0.0f;
        b.byte = (uint8_t)(e + 127);
    } else {
        const float amax = __builtin_bit_cast(float, amax_bits);
        b.pre = e4m3_prescale(amax_bits);
        b.inv = e4m3_inverse_scale(amax, b.pre);
        b.scale = e4m3_scale(amax);
        b.byte = 0;
    }
    return b;
}
// Entry idx of a scale array: fp32 scales, or E8M0 bytes for MX.
__device__ __forceinline__ void store_block_scale(void* scales, size_t idx, const BlockScale& b, bool mx) {
    if (mx)
        static_cast<uint8_t*>(scales)[idx] = b.byte;
    else
        static_cast<float*>(scales)[idx] = b.scale;
}

// The 8 codes of (f[0..7] * pre) * inv, in memory order (the first product
// is exact: pre is a power of two that keeps every value finite).
__device__ __forceinline__ u32x2 quantize8_e4m3(const float (&f)[8], float inv, float pre = 1.0f) {
    u32x2 codes;
    const auto q = [&](int i) { return clamp448((f[i] * pre) * inv); };
#pragma unroll
    for (int w = 0; w < 2; ++w) {
        int packed = __builtin_amdgcn_cvt_pk_fp8_f32(q(4 * w), q(4 * w + 1), 0, false);
        packed = __builtin_amdgcn_cvt_pk_fp8_f32(q(4 * w + 2), q(4 * w + 3), packed, true);
        codes[w] = (uint32_t)packed;
    }
    return codes;
}

}  // namespace moe
