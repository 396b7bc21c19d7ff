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

#include <algorithm>

namespace moe {
namespace {

constexpr int kThreads = 256;
constexpr int kKMax = 16;

template <int U, bool ROW_PER_WAVE, int KC>
__global__ __launch_bounds__(kThreads) void expand_rows_kernel(const u32x4* __restrict__ x,
                                                               const int32_t* __restrict__ dest_of_src, uint32_t n,
                                                               uint32_t H16, FastDiv div_h16, int k_arg,
                                                               u32x4* __restrict__ x_exp) {
    const int k = KC > 0 ? KC : k_arg;  // fixed: the k row indices come in under one wait
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
    // k fixed at compile time lets a wave issue its k stores back to back
    // instead of one per index fetch: 30.4 -> 28.0 us at T x H = 4096 x
    // 2048 (k = 8), but 10.7 -> 11.0 us at 1023 x 4096 (k = 6) and 213.7 ->
    // 222 us at 8192 x 7168 (k = 8), where more write streams at once cost
    // more than the fetches; so only for rows up to 2048 columns.
    const bool row = H16 % kWave == 0;
    const bool fixed_k = row && H16 <= 256;
    if (fixed_k && k == 8)
        expand_rows_kernel<U, true, 8><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, dv, k, xo);
    else if (fixed_k && k == 6)
        expand_rows_kernel<U, true, 6><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, dv, k, xo);
    else if (fixed_k && k == 4)
        expand_rows_kernel<U, true, 4><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, dv, k, xo);
    else if (fixed_k && k == 2)
        expand_rows_kernel<U, true, 2><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, dv, k, xo);
    else if (row)
        expand_rows_kernel<U, true, 0><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, dv, k, xo);
    else
        expand_rows_kernel<U, false, 0><<<blocks, kThreads, 0, stream>>>(xs, dest_of_src, n, H16, dv, k, xo);
    return hipGetLastError();
}

// ----------------------------------------------------------- grouped form
// Destination-row order, from the route's row list.  Writing in token order
// sends every token's k rows to k experts' segments at once, i.e. E open write
// streams across the whole output; in destination order the writes of the
// whole chip stay inside one moving window, which HBM absorbs faster.  The
// price is that each source row is read k times -- so the tokens are split
// into groups (RowGroups) and the rows of one group are copied by one XCD:
// workgroup b runs on XCD b % 8 and copies rows of group (m / chunks) * 8 +
// b % 8, m = b / 8, in destination order.  While an XCD works on a group, the
// group's source rows stay in its L2 and HBM sees each read about once; the
// eight XCDs work on neighbouring groups, whose rows in each expert segment
// are neighbours too.  Each workgroup copies kGroupedItems / (H/8) rows (at
// least one): one vector per lane in two passes, or four vectors per lane
// in one pass when a row is wider than kGroupedItems vectors (at H = 7168
// the 896 vectors of a row then take one pass instead of two: 217 -> 209 us
// for the DeepSeek-V3 batch in a standalone probe; 213 -> 216 us with two
// per lane).  On the narrower rows one vector per lane beat two (8192 x
// 2048: 63.2 -> 61.1 us per call; 8192 x 4096, k = 6: 90.3 -> 88.9).
//
// A group's first rows in destination order need source rows all over the
// group, so when x comes from HBM (not from the Infinity Cache) the early
// workgroups of a group each wait for their own misses.  So workgroup c of a
// group first issues cached loads of the group's source vectors
// [c*kGroupedPrefetch*256, (c+1)*kGroupedPrefetch*256): the group's first
// workgroups pull its whole source (2 MiB at most) into the XCD's L2 at
// streaming speed, and the rest hit.  A group has one workgroup per listed
// row pair (or row), so the slices cover its whole source whenever
// H/8 <= 1024 k (at rows <= 512 vectors they cover it 2k times over); past
// that only a part is warmed, which costs time, not correctness.  Loads
// outside the group are skipped.  Measured at the Qwen3-30B-A3B shape with x
// in HBM: 27.0 -> 23.0 us (4 vectors per lane; 24.4 with 1, 23.1 with 2).
constexpr int kGroupedThreads = 256;
constexpr int kGroupedItems = 512;  // 16-byte vectors per workgroup: small windows
constexpr int kGroupedPrefetch = 4;  // source vectors per lane touched up front

// Copy `items` vectors of the listed rows lst[0..items / H16) in list order.
template <int U>
__device__ __forceinline__ void copy_group_rows(const u32x4* __restrict__ x, const int2* __restrict__ lst,
                                                uint32_t items, uint32_t H16, FastDiv div_h16,
                                                u32x4* __restrict__ x_exp) {
    for (uint32_t i0 = threadIdx.x; i0 < items; i0 += kGroupedThreads * U) {
        int2 ent[U];
        uint32_t col[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = min(i0 + u * kGroupedThreads, items - 1);  // clamped: loads stay in bounds
            const uint32_t r = fastdiv(i, div_h16);
            col[u] = i - r * H16;
            ent[u] = lst[r];
        }
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) v[u] = x[(size_t)ent[u].y * H16 + col[u]];  // cached: reused from L2
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * kGroupedThreads < items) store_stream(x_exp + (size_t)ent[u].x * H16 + col[u], v[u]);
        // an unconditional use of every vector: otherwise the compiler sinks
        // a vector's row-list and source loads into its store's branch, where
        // they wait for all older loads and then for each other
#pragma unroll
        for (int u = 0; u < U; ++u) asm volatile("" ::"v"(v[u][0]));
    }
}

template <int U>
__global__ __launch_bounds__(kGroupedThreads) void expand_grouped_kernel(const u32x4* __restrict__ x,
                                                                         const int2* __restrict__ row_list,
                                                                         RowGroups groups, int k, uint32_t H16,
                                                                         FastDiv div_h16, uint32_t rows_per_wg,
                                                                         uint32_t chunks,
                                                                         u32x4* __restrict__ x_exp) {
    const uint32_t m = blockIdx.x / kXcds;
    const int g = (int)(m / chunks) * kXcds + (int)(blockIdx.x % kXcds);
    if (g >= groups.n) return;
    const uint32_t chunk = m % chunks;
    const uint32_t first = chunk * rows_per_wg;
    const int32_t t0 = group_tok(groups, g);
    const int32_t t1 = group_tok(groups, g + 1);
    // this workgroup's slice of the group's source vectors, into L2
    const u32x4* src = x + (size_t)t0 * H16;
    const size_t src_n = (size_t)(t1 - t0) * H16;
    const size_t pf0 = (size_t)chunk * (kGroupedThreads * kGroupedPrefetch) + threadIdx.x;
    u32x4 warm[kGroupedPrefetch];
#pragma unroll
    for (int p = 0; p < kGroupedPrefetch; ++p) {
        const size_t j = pf0 + (size_t)p * kGroupedThreads;
        warm[p] = j < src_n ? src[j] : (u32x4){0u, 0u, 0u, 0u};
    }
    const uint32_t n = (uint32_t)(t1 - t0) * (uint32_t)k;
    if (first < n) copy_group_rows<U>(x, row_list + (size_t)t0 * k + first, min(rows_per_wg, n - first) * H16, H16,
                                      div_h16, x_exp);
    // the touched vectors are not needed: an empty use keeps the loads (the
    // compiler narrows them to one dword per vector, which still brings in
    // every line of the slice)
#pragma unroll
    for (int p = 0; p < kGroupedPrefetch; ++p) asm volatile("" ::"v"(warm[p][0]));
}

}  // namespace

hipError_t launch_expand_grouped(const void* x, const int32_t* row_list, const RowGroups& groups, int H, int k,
                                 void* x_expanded, hipStream_t stream) {
    const uint32_t H16 = (uint32_t)H / 8;
    const uint32_t rows_per_wg = H16 >= (uint32_t)kGroupedItems ? 1u : (uint32_t)kGroupedItems / H16;
    uint32_t chunks = 0;  // workgroups per group
    for (int g = 0; g < groups.n; ++g) {
        const uint32_t n = (uint32_t)(group_tok(groups, g + 1) - group_tok(groups, g)) * (uint32_t)k;
        chunks = std::max(chunks, (n + rows_per_wg - 1) / rows_per_wg);
    }
    if (chunks == 0) return hipSuccess;
    const uint32_t rounds = ((uint32_t)groups.n + kXcds - 1) / kXcds;  // groups per XCD
    const dim3 grid(rounds * kXcds * chunks);
    const u32x4* xs = static_cast<const u32x4*>(x);
    const int2* lst = reinterpret_cast<const int2*>(row_list);
    u32x4* xo = static_cast<u32x4*>(x_expanded);
    if (H16 > (uint32_t)kGroupedItems)
        expand_grouped_kernel<4><<<grid, kGroupedThreads, 0, stream>>>(xs, lst, groups, k, H16, make_fastdiv(H16),
                                                                       rows_per_wg, chunks, xo);
    else  // one vector per lane, two passes: 63.2 -> 61.1 us per call at 8192 x 2048 against two per lane
        expand_grouped_kernel<1><<<grid, kGroupedThreads, 0, stream>>>(xs, lst, groups, k, H16, make_fastdiv(H16),
                                                                       rows_per_wg, chunks, xo);
    return hipGetLastError();
}

hipError_t launch_expand_rows(const void* x, const int32_t* dest_of_src, int T, int H, int k, void* x_expanded,
                              hipStream_t stream) {
    // one vector per lane keeps more workgroups in flight on small batches,
    // and on very large ones it also won (8192 x 7168: 214.6 -> 204.0 us,
    // 4096 x 7168: 109.9 -> 105.1, 16384 x 2048: 125.6 -> 124.7); between,
    // two per lane (4096 x 2048: 27.9 against 29.8 us; 2048 x 7168: 51.4
    // against 52.0; 8192 x 2048: 59.9 against 61.4)
    const size_t n = (size_t)T * (H / 8);
    if (n < (size_t)256 * kThreads * 2 || n >= ((size_t)3 << 20))
        return launch_u<1>(x, dest_of_src, T, H, k, x_expanded, stream);
    return launch_u<2>(x, dest_of_src, T, H, k, x_expanded, stream);
}

}  // namespace moe
