// moe_combine on gfx950: the weighted accumulation of each token's k expert
// outputs back into token order ("CuTeDSL at Perplexity", MoE
// dispatch/combine: accumulation in registers, vectorised, using the
// positions dispatch computed).
//
// Token-major gather: a work item is one lane vector (16 bytes = 8 bf16, or
// 8 bytes = 4 bf16) of one output token row; items are numbered row-major
// over [T, H/8] (or [T, H/4]).  The lane issues the k loads of its column
// from the k expert rows at once (k independent loads in flight),
// accumulates w_j * y_j in fp32 in j order in registers and stores one
// rounded vector.  No atomics, so the result is deterministic.  When a row
// is a whole number of waves the token index is wave-uniform and its k
// weights and k row indices come in by scalar loads.
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

// One wave per workgroup: measured against 128 and 256 lanes with rotating
// input sets (T x H = 4096 x 2048: 26.6 -> 25.9 us; 8192 x 7168: 185.7 ->
// 180.2 us; 1023 x 4096: 14.6 -> 14.3 us).
constexpr int kThreads = 64;
constexpr int kKMax = 16;

template <int W>
struct LaneVec;
template <>
struct LaneVec<4> {
    typedef u32x4 type;
};
template <>
struct LaneVec<2> {
    typedef u32x2 type;
};

// The lane's output vector, non-temporal; the 8-byte lanes also set sc1:
// in the path at T x H = 4096 x 2048 combine 26.1 -> 25.8 us, at 8192 x 7168
// 173.2 -> 172.4 us (HIP events, medians of 200 steps, the two forms
// alternated four times; sc0 on top changes nothing), while the 16-byte lanes
// of a 1023 x 4096 batch lose 0.1 us with it.
template <int W>
__device__ __forceinline__ void store_out(typename LaneVec<W>::type* __restrict__ out, uint32_t i, uint32_t n,
                                          const typename LaneVec<W>::type& o) {
    if constexpr (W == 2)
        store_stream_sc1(out, blockIdx.x * kThreads, i, n, o);  // one wave per workgroup
    else
        __builtin_nontemporal_store(o, out + i);
}

// W words (2W bf16) per lane.
template <bool ROW_PER_WAVE, int KC, int W>
__global__ __launch_bounds__(kThreads) void combine_kernel(const typename LaneVec<W>::type* __restrict__ y,
                                                           const float* __restrict__ w,
                                                           const int32_t* __restrict__ dest_of_src, uint32_t n,
                                                           uint32_t HL, FastDiv div_hl, int k_arg,
                                                           typename LaneVec<W>::type* __restrict__ out) {
    typedef typename LaneVec<W>::type Vec;
    const int k = KC > 0 ? KC : k_arg;
    const uint32_t i = blockIdx.x * kThreads + threadIdx.x;
    if (i >= n) return;
    uint32_t t = fastdiv(i, div_hl);
    if constexpr (ROW_PER_WAVE) t = uniform(t);
    const uint32_t c = i - t * HL;
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
    Vec v[kKMax];
#pragma unroll
    for (int j = 0; j < kKMax; ++j)
        if (j < k) v[j] = __builtin_nontemporal_load(y + (size_t)dj[j] * HL + c);
    float acc[2 * W];
#pragma unroll
    for (int e = 0; e < 2 * W; ++e) acc[e] = 0.f;
#pragma unroll
    for (int j = 0; j < kKMax; ++j) {
        if (j < k) {
#pragma unroll
            for (int q = 0; q < W; ++q) {
                acc[2 * q] = __builtin_fmaf(wj[j], bf16_lo(v[j][q]), acc[2 * q]);
                acc[2 * q + 1] = __builtin_fmaf(wj[j], bf16_hi(v[j][q]), acc[2 * q + 1]);
            }
        }
    }
    Vec o;
#pragma unroll
    for (int q = 0; q < W; ++q) o[q] = pack_bf16x2(acc[2 * q], acc[2 * q + 1]);
    store_out<W>(out, i, n, o);
}

template <bool ROW_PER_WAVE, int KC, int W>
void launch_w(const void* y, const float* topk_weights, const int32_t* dest_of_src, int T, int H, int k, void* out,
              hipStream_t stream) {
    typedef typename LaneVec<W>::type Vec;
    const uint32_t HL = (uint32_t)H / (2 * W);
    const uint32_t n = (uint32_t)T * HL;
    const uint32_t blocks = (n + kThreads - 1) / kThreads;
    combine_kernel<ROW_PER_WAVE, KC, W><<<blocks, kThreads, 0, stream>>>(
        static_cast<const Vec*>(y), topk_weights, dest_of_src, n, HL, make_fastdiv(HL), k, static_cast<Vec*>(out));
}

template <int KC>
void launch_kc(bool narrow, const void* y, const float* topk_weights, const int32_t* dest_of_src, int T, int H, int k,
               void* out, hipStream_t stream) {
    if (narrow)
        launch_w<true, KC, 2>(y, topk_weights, dest_of_src, T, H, k, out, stream);
    else
        launch_w<true, KC, 4>(y, topk_weights, dest_of_src, T, H, k, out, stream);
}

}  // namespace

hipError_t launch_combine(const void* y, const float* topk_weights, const int32_t* dest_of_src, int T, int H,
                          int k, void* out, hipStream_t stream) {
    const uint32_t H16 = (uint32_t)H / 8;
    // 8-byte lanes (twice the waves, half the bytes each) from 2^18 16-byte
    // items: 25.2 -> 24.6 us at T x H = 4096 x 2048 and 180.2 -> 175.0 us at
    // 8192 x 7168 in a back-to-back probe; at 1024 x 4096 they first lost
    // (13.6 -> 14.4 us), but with the sc1 stores the 1023 x 4096 batch (k = 6)
    // gains in the path, 11.78 -> 11.54 us.  Only for the fixed-k kernels with
    // rows of whole 8-byte waves, and while the 8-byte item count stays below
    // 2^31 (the range of the row division).
    const bool row = H16 % kWave == 0;
    const uint64_t items16 = (uint64_t)T * H16;
    const bool narrow = (uint32_t)H % (4 * kWave) == 0 && items16 >= (1u << 18) && items16 < (1u << 30);
    if (row && k == 8)
        launch_kc<8>(narrow, y, topk_weights, dest_of_src, T, H, k, out, stream);
    else if (row && k == 6)
        launch_kc<6>(narrow, y, topk_weights, dest_of_src, T, H, k, out, stream);
    else if (row && k == 4)
        launch_kc<4>(narrow, y, topk_weights, dest_of_src, T, H, k, out, stream);
    else if (row && k == 2)
        launch_kc<2>(narrow, y, topk_weights, dest_of_src, T, H, k, out, stream);
    else if (row)
        launch_w<true, 0, 4>(y, topk_weights, dest_of_src, T, H, k, out, stream);
    else
        launch_w<false, 0, 4>(y, topk_weights, dest_of_src, T, H, k, out, stream);
    return hipGetLastError();
}

}  // namespace moe
