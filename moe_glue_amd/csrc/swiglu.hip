// moe_swiglu on gfx950: doActivation (FlashInfer PR analysis, sections 1-2)
// -- gated SiLU over the first grouped GEMM's output.
//
// The page's fix for this kernel sizes the threads of a row to the
// intermediate size (a fixed 256 threads per row idled most warps at I=768)
// and sizes the grid per SM.  On wave64 the natural form of that idea is to
// drop the per-row thread block altogether: a work item is one 16-byte vector
// of 8 outputs, items are numbered row-major over [R, I/8] and lanes take
// consecutive items, so no lane idles whatever I is (I=768 gives 96 items
// per row; 2 rows fill 3 waves exactly).  Each item reads 16 B of gate and
// 16 B of up and writes 16 B; on the largest batches items are 8-byte
// vectors of 4 outputs instead (launch_swiglu).
//
// Arithmetic: silu(g) * u in fp32 with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32), one round-to-nearest-even conversion per output
// (v_cvt_pk_bf16_f32).
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// One wave per workgroup: measured against 128-1024 lanes with 24 rotating
// input sets, the smallest workgroups finish the grid soonest (R x I =
// 32768 x 768: 24.8 -> 24.3 us; 65536 x 2048: 124.7 -> 118.7 us; 6138 x
// 1408: 10.0 -> 9.8 us; 256 x 768 unchanged).
constexpr int kThreads = 64;

__device__ __forceinline__ float silu_mul(float g, float u) {
    // g / (1 + e^-g); e^-g = 2^(-g * log2 e).  For g << 0 the exponential is
    // +inf and the quotient is -0; for g >> 0 it is 0 and the quotient is g.
    const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
    return g * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

template <int U>
__global__ __launch_bounds__(kThreads) void swiglu_kernel(const u32x4* __restrict__ h, uint32_t n, uint32_t I8,
                                                          FastDiv div_i8, u32x4* __restrict__ act) {
    const uint32_t base = blockIdx.x * (kThreads * U) + threadIdx.x;
    u32x4 gv[U], uv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i = base + u * kThreads;
        if (i < n) {
            const uint32_t r = fastdiv(i, div_i8);
            const size_t gi = (size_t)r * (2 * I8) + (i - r * I8);
            gv[u] = load_stream(h + gi);
            uv[u] = load_stream(h + gi + I8);
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i = base + u * kThreads;
        if (i < n) {
            float g[8], up[8], o[8];
            unpack8(gv[u], g);
            unpack8(uv[u], up);
#pragma unroll
            for (int e = 0; e < 8; ++e) o[e] = silu_mul(g[e], up[e]);
            store_stream(act + i, pack8(o));
        }
    }
}

// 8-byte lanes: 4 outputs per item, items row-major over [R, I/4]; the
// stores carry sc1 beside nt (one wave per workgroup).
__global__ __launch_bounds__(kThreads) void swiglu8_kernel(const u32x2* __restrict__ h, uint32_t n, uint32_t I4,
                                                           FastDiv div_i4, u32x2* __restrict__ act) {
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    const uint32_t r = fastdiv(i, div_i4);
    const size_t gi = (size_t)r * (2 * I4) + (i - r * I4);
    const u32x2 gv = __builtin_nontemporal_load(h + gi);
    const u32x2 uv = __builtin_nontemporal_load(h + gi + I4);
    u32x2 o;
#pragma unroll
    for (int q = 0; q < 2; ++q)
        o[q] = pack_bf16x2(silu_mul(bf16_lo(gv[q]), bf16_lo(uv[q])), silu_mul(bf16_hi(gv[q]), bf16_hi(uv[q])));
    store_stream_sc1(act, blockIdx.x * kThreads, i, n, o);
}

template <int U>
hipError_t launch_u(const void* h, int R, int I, void* act, hipStream_t stream) {
    const uint32_t I8 = (uint32_t)I / 8;
    const uint32_t n = (uint32_t)R * I8;
    const uint32_t blocks = (n + kThreads * U - 1) / (kThreads * U);
    swiglu_kernel<U><<<blocks, kThreads, 0, stream>>>(static_cast<const u32x4*>(h), n, I8, make_fastdiv(I8),
                                                      static_cast<u32x4*>(act));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_swiglu(const void* h, int R, int I, void* act, hipStream_t stream) {
    // From 2^23 16-byte items, 8-byte lanes with sc1 stores: R x I = 65536 x
    // 2048 119.9 -> 117.2 us, 32768 x 2048 61.6 -> 60.4, 131072 x 768 92.4 ->
    // 90.5 (HIP events in the path, medians of 200 steps, p90 lower too).
    // Below that (32768 x 768, 65536 x 768) the median gains a little but the
    // step times spread (p90 26.0 -> 28.6 and 49.5 -> 55 us), so those keep
    // 16-byte lanes.  The 8-byte item count stays below 2^31 (row division).
    const uint64_t items16 = (uint64_t)R * ((uint32_t)I / 8);
    if (items16 >= (1u << 23) && items16 < (1u << 29)) {
        const uint32_t I4 = (uint32_t)I / 4;
        const uint32_t n = (uint32_t)R * I4;
        swiglu8_kernel<<<(n + kThreads - 1) / kThreads, kThreads, 0, stream>>>(
            static_cast<const u32x2*>(h), n, I4, make_fastdiv(I4), static_cast<u32x2*>(act));
        return hipGetLastError();
    }
    // Otherwise one 16-byte item per lane: faster than two at the
    // Qwen3-30B-A3B shape (27.1 vs 28.4 us for 151 MB, interleaved A/B): more
    // workgroups in flight beat more loads per lane here.
    return launch_u<1>(h, R, I, act, stream);
}

}  // namespace moe
