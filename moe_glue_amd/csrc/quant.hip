// moe_expand_rows_fp8 on gfx950: the expand step with FP8 quantisation fused
// between its load and its store (the FlashInfer PR analysis shows an
// operation in that place in expandInputRowsKernel; "CuTeDSL at Perplexity",
// Blackwell support, adapts its kernels to FP8 block-wise scaling with
// absolute maxima over small groups of elements).
//
// Same work items as the bf16 expand: one 16-byte vector (8 bf16) of one token
// row per lane, token-major, so x is read once.  The vector is quantised as in
// fp8_common.h (group absolute maximum over group/8 lanes, OCP E4M3 codes);
// the 8 codes (8 bytes) are stored to each of the token's k expanded rows, and
// the group's first lane stores its scale k times.  HBM traffic: T*H*2 read,
// R*H + R*(H/group)*4 written -- about 0.57x the bf16 expand at group 128.
// The MXFP8 form below differs only in its scale: a power of two per block of
// 32 columns, stored as one E8M0 byte.
#include "device_common.h"
#include "fp8_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kKMax = 16;

template <int GL, bool ROW_PER_WAVE>
__global__ __launch_bounds__(kThreads) void expand_rows_fp8_kernel(const u32x4* __restrict__ x,
                                                                   const int32_t* __restrict__ dest_of_src, uint32_t n,
                                                                   uint32_t H16, FastDiv div_h16, int k, uint32_t G,
                                                                   u32x2* __restrict__ q_out,
                                                                   float* __restrict__ scales) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    // Every lane of a wave takes part in the group reduction; lanes past the
    // end work on zeros (n is a multiple of GL, so no group straddles the end).
    const bool live = i < n;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) v = load_stream(x + i);
    float f[8];
    unpack8(v, f);
    const uint32_t amax_bits = group_reduce<GL, Op::Max>(abs_max_bits8(f));
    if (!live) return;
    const float amax = __builtin_bit_cast(float, amax_bits);
    const float scale = e4m3_scale(amax);
    const float pre = e4m3_prescale(amax_bits);
    const u32x2 codes = quantize8_e4m3(f, e4m3_inverse_scale(amax, pre), pre);
    uint32_t t = fastdiv(i, div_h16);
    if constexpr (ROW_PER_WAVE) t = uniform(t);
    const uint32_t c = i - t * H16;
    const int32_t* d = dest_of_src + (size_t)t * k;
    int32_t dj[kKMax];
#pragma unroll
    for (int j = 0; j < kKMax; ++j) dj[j] = d[j < k ? j : k - 1];
    const bool first_of_group = (threadIdx.x % GL) == 0;
    const uint32_t g = c / GL;
#pragma unroll
    for (int j = 0; j < kKMax; ++j) {
        if (j < k) {
            __builtin_nontemporal_store(codes, q_out + (size_t)dj[j] * H16 + c);
            if (first_of_group) scales[(size_t)dj[j] * G + g] = scale;
        }
    }
}

// MXFP8 (OCP microscaling; "CuTeDSL at Perplexity", Blackwell support, takes
// the MXFP8 absolute maximum over 32 elements): a block of 32 columns is 4
// consecutive lanes.  Its scale is the power of two 2^e of fp8_common.h's
// mx_scale_exponent, stored as the E8M0 byte e + 127; the codes are
// E4M3(clamp(x * 2^-e, +-448)), and multiplying by a power of two is exact.
constexpr int kMxLanes = 4;  // 32 columns / 8 per lane

template <bool ROW_PER_WAVE>
__global__ __launch_bounds__(kThreads) void expand_rows_mxfp8_kernel(const u32x4* __restrict__ x,
                                                                     const int32_t* __restrict__ dest_of_src,
                                                                     uint32_t n, uint32_t H16, FastDiv div_h16, int k,
                                                                     uint32_t B, u32x2* __restrict__ q_out,
                                                                     uint8_t* __restrict__ scales) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    // every lane takes part in the block reduction; n is a multiple of 4, so
    // no block straddles the end and lanes past it work on zeros
    const bool live = i < n;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (live) v = load_stream(x + i);
    float f[8];
    unpack8(v, f);
    const uint32_t amax_bits = group_reduce<kMxLanes, Op::Max>(abs_max_bits8(f));
    if (!live) return;
    const int e = mx_scale_exponent(amax_bits);
    const float inv = mx_inverse_scale(e);
    const uint8_t byte = (uint8_t)(e + 127);
    const u32x2 codes = quantize8_e4m3(f, inv);
    uint32_t t = fastdiv(i, div_h16);
    if constexpr (ROW_PER_WAVE) t = uniform(t);
    const uint32_t c = i - t * H16;
    const int32_t* d = dest_of_src + (size_t)t * k;
    int32_t dj[kKMax];
#pragma unroll
    for (int j = 0; j < kKMax; ++j) dj[j] = d[j < k ? j : k - 1];
    const bool first_of_block = (threadIdx.x % kMxLanes) == 0;
    const uint32_t b = c / kMxLanes;
#pragma unroll
    for (int j = 0; j < kKMax; ++j) {
        if (j < k) {
            __builtin_nontemporal_store(codes, q_out + (size_t)dj[j] * H16 + c);
            if (first_of_block) scales[(size_t)dj[j] * B + b] = byte;
        }
    }
}

template <int GL>
hipError_t launch_gl(const void* x, const int32_t* dest_of_src, int T, int H, int k, int group, void* q_out,
                     float* scales, hipStream_t stream) {
    const uint32_t H16 = (uint32_t)H / 8;
    const uint32_t n = (uint32_t)T * H16;
    const uint32_t blocks = (n + kThreads - 1) / kThreads;
    const uint32_t G = (uint32_t)(H / group);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x2* q = static_cast<u32x2*>(q_out);
    if (H16 % kWave == 0)
        expand_rows_fp8_kernel<GL, true><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16,
                                                                          make_fastdiv(H16), k, G, q, scales);
    else
        expand_rows_fp8_kernel<GL, false><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16,
                                                                           make_fastdiv(H16), k, G, q, scales);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expand_rows_mxfp8(const void* x, const int32_t* dest_of_src, int T, int H, int k, void* q_out,
                                    uint8_t* scales, hipStream_t stream) {
    const uint32_t H16 = (uint32_t)H / 8;
    const uint32_t n = (uint32_t)T * H16;
    const uint32_t blocks = (n + kThreads - 1) / kThreads;
    const uint32_t B = (uint32_t)(H / 32);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x2* q = static_cast<u32x2*>(q_out);
    if (H16 % kWave == 0)
        expand_rows_mxfp8_kernel<true><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, make_fastdiv(H16), k,
                                                                        B, q, scales);
    else
        expand_rows_mxfp8_kernel<false><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, make_fastdiv(H16),
                                                                         k, B, q, scales);
    return hipGetLastError();
}

hipError_t launch_expand_rows_fp8(const void* x, const int32_t* dest_of_src, int T, int H, int k, int group,
                                  void* q_out, float* scales, hipStream_t stream) {
    switch (group / 8) {
        case 1: return launch_gl<1>(x, dest_of_src, T, H, k, group, q_out, scales, stream);
        case 2: return launch_gl<2>(x, dest_of_src, T, H, k, group, q_out, scales, stream);
        case 4: return launch_gl<4>(x, dest_of_src, T, H, k, group, q_out, scales, stream);
        case 8: return launch_gl<8>(x, dest_of_src, T, H, k, group, q_out, scales, stream);
        case 16: return launch_gl<16>(x, dest_of_src, T, H, k, group, q_out, scales, stream);
        case 32: return launch_gl<32>(x, dest_of_src, T, H, k, group, q_out, scales, stream);
        default: return launch_gl<64>(x, dest_of_src, T, H, k, group, q_out, scales, stream);
    }
}

}  // namespace moe
