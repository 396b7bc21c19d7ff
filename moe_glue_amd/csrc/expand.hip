// moe_expand_rows on gfx950: expandInputRows (FlashInfer PR analysis,
// section 1) -- copy every token row into its k expert-contiguous rows.
//
// Token-major: each 16-byte vector of x is read once and stored k times, so
// HBM sees the algorithmic minimum (T*H*2 read, T*k*H*2 written).  A gather
// ordered by destination row would read every source row k times instead.
//
// Work item = one 16-byte vector (8 bf16) of one token row; items are
// numbered row-major over [T, H/8], so the load address is the item index
// itself.  Each lane takes U items spaced one workgroup-width apart, so every
// wave touches 64 consecutive vectors per access (1 KiB, fully coalesced) and
// each lane has U independent loads in flight.  When a row is a whole number
// of waves (H/8 % 64 == 0) the token index is wave-uniform and the k
// destination rows are fetched with scalar loads.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kKMax = 16;

template <int U, bool ROW_PER_WAVE>
__global__ __launch_bounds__(kThreads) void expand_rows_kernel(const u32x4* __restrict__ x,
                                                               const int32_t* __restrict__ dest_of_src, uint32_t n,
                                                               uint32_t H16, FastDiv div_h16, int k,
                                                               u32x4* __restrict__ x_exp) {
    const uint32_t base = blockIdx.x * (kThreads * U) + threadIdx.x;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i = base + u * kThreads;
        if (i < n) v[u] = load_stream(x + i);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const uint32_t i = base + u * kThreads;
        if (i < n) {
            uint32_t t = fastdiv(i, div_h16);
            if constexpr (ROW_PER_WAVE) t = uniform(t);
            const uint32_t c = i - t * H16;
            const int32_t* d = dest_of_src + (size_t)t * k;
            // all k row indices first (clamped: unconditional, in bounds), then the stores
            int32_t dj[kKMax];
#pragma unroll
            for (int j = 0; j < kKMax; ++j) dj[j] = d[j < k ? j : k - 1];
#pragma unroll
            for (int j = 0; j < kKMax; ++j)
                if (j < k) store_stream(x_exp + (size_t)dj[j] * H16 + c, v[u]);
        }
    }
}

template <int U>
hipError_t launch_u(const void* x, const int32_t* dest_of_src, int T, int H, int k, void* x_exp,
                    hipStream_t stream) {
    const uint32_t H16 = (uint32_t)H / 8;
    const uint32_t n = (uint32_t)T * H16;
    const uint32_t blocks = (n + kThreads * U - 1) / (kThreads * U);
    const FastDiv dv = make_fastdiv(H16);
    const u32x4* xs = static_cast<const u32x4*>(x);
    u32x4* xo = static_cast<u32x4*>(x_exp);
    if (H16 % kWave == 0)
        expand_rows_kernel<U, true><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, dv, k, xo);
    else
        expand_rows_kernel<U, false><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, dv, k, xo);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_expand_rows(const void* x, const int32_t* dest_of_src, int T, int H, int k, void* x_expanded,
                              hipStream_t stream) {
    // small batches: one vector per lane keeps more workgroups in flight
    const size_t n = (size_t)T * (H / 8);
    if (n < (size_t)256 * kThreads * 2) return launch_u<1>(x, dest_of_src, T, H, k, x_expanded, stream);
    return launch_u<2>(x, dest_of_src, T, H, k, x_expanded, stream);
}

}  // namespace moe
