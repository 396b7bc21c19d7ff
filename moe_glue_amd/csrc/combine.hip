// moe_combine on gfx950: the weighted accumulation of each token's k expert
// outputs back into token order ("CuTeDSL at Perplexity", MoE
// dispatch/combine: accumulation in registers, vectorised, using the
// positions dispatch computed).
//
// Token-major gather: a work item is one 16-byte vector (8 bf16) of one output
// token row; items are numbered row-major over [T, H/8].  The lane issues the
// k 16-byte loads of its column from the k expert rows at once (k independent
// loads in flight), accumulates w_j * y_j in fp32 in j order in registers and
// stores one rounded 16-byte vector.  No atomics, so the result is
// deterministic.  When a row is a whole number of waves the token index is
// wave-uniform and its k weights and k row indices come in by scalar loads.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// One wave per workgroup: measured against 128 and 256 lanes with rotating
// input sets (T x H = 4096 x 2048: 26.6 -> 25.9 us; 8192 x 7168: 185.7 ->
// 180.2 us; 1023 x 4096: 14.6 -> 14.3 us).
constexpr int kThreads = 64;
constexpr int kKMax = 16;

template <bool ROW_PER_WAVE, int KC>
__global__ __launch_bounds__(kThreads) void combine_kernel(const u32x4* __restrict__ y,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ dest_of_src, uint32_t n,
                                                           uint32_t H16, FastDiv div_h16, int k_arg,
                                                           u32x4* __restrict__ out) {
    const int k = KC > 0 ? KC : k_arg;
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    uint32_t t = fastdiv(i, div_h16);
    if constexpr (ROW_PER_WAVE) t = uniform(t);
    const uint32_t c = i - t * H16;
    const int32_t* d = dest_of_src + (size_t)t * k;
    const float* wt = w + (size_t)t * k;

    // Fetch all k row indices and weights before the first row load.  With k
    // fixed at compile time (KC: the common 2, 4, 6 and 8 with whole-wave
    // rows) they come in as two scalar loads under one wait and the k row
    // loads follow back to back (27.0 -> 26.5 us at T x H = 4096 x 2048,
    // k = 8; 44 registers instead of 74).  For another k the clamped index
    // keeps every fetch in bounds, but the compiler issues each one inside
    // its row's branch, one wait per row.
    int32_t dj[kKMax];
    float wj[kKMax];
#pragma unroll
    for (int j = 0; j < kKMax; ++j) {
        const int jj = j < k ? j : k - 1;
        dj[j] = d[jj];
        wj[j] = wt[jj];
    }
    u32x4 v[kKMax];
#pragma unroll
    for (int j = 0; j < kKMax; ++j)
        if (j < k) v[j] = load_stream(y + (size_t)dj[j] * H16 + c);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kKMax; ++j) {
        if (j < k) {
            float f[8];
            unpack8(v[j], f);
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[e] = __builtin_fmaf(wj[j], f[e], acc[e]);
        }
    }
    store_stream(out + i, pack8(acc));
}

}  // namespace

hipError_t launch_combine(const void* y, const float* topk_weights, const int32_t* dest_of_src, int T, int H,
                          int k, void* out, hipStream_t stream) {
    const uint32_t H16 = (uint32_t)H / 8;
    const uint32_t n = (uint32_t)T * H16;
    const uint32_t blocks = (n + kThreads - 1) / kThreads;
    const FastDiv dv = make_fastdiv(H16);
    const u32x4* ys = static_cast<const u32x4*>(y);
    u32x4* o = static_cast<u32x4*>(out);
    const bool row = H16 % kWave == 0;
    if (row && k == 8)
        combine_kernel<true, 8><<<blocks, kThreads, 0, stream>>>(ys, topk_weights, dest_of_src, n, H16, dv, k, o);
    else if (row && k == 6)
        combine_kernel<true, 6><<<blocks, kThreads, 0, stream>>>(ys, topk_weights, dest_of_src, n, H16, dv, k, o);
    else if (row && k == 4)
        combine_kernel<true, 4><<<blocks, kThreads, 0, stream>>>(ys, topk_weights, dest_of_src, n, H16, dv, k, o);
    else if (row && k == 2)
        combine_kernel<true, 2><<<blocks, kThreads, 0, stream>>>(ys, topk_weights, dest_of_src, n, H16, dv, k, o);
    else if (row)
        combine_kernel<true, 0><<<blocks, kThreads, 0, stream>>>(ys, topk_weights, dest_of_src, n, H16, dv, k, o);
    else
        combine_kernel<false, 0><<<blocks, kThreads, 0, stream>>>(ys, topk_weights, dest_of_src, n, H16, dv, k, o);
    return hipGetLastError();
}

}  // namespace moe
