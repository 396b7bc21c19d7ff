// moe_route_expand for small batches on gfx950: routing and the expansion of
// the token rows in ONE launch.
//
// "CuTeDSL at Perplexity" (Grid synchronization; MoE dispatch/combine > Local)
// describes the decode dispatch as one block that reads the routing
// information and then signals the rest of the grid, whose blocks copy token
// chunks -- a grid barrier, because a second launch costs about as much.  On
// this part a cooperative launch and its grid barrier cost far more than a
// launch, and a plain launch gives no co-residency guarantee for spinning on a
// flag.  So no workgroup waits for another: for a small batch (T <= 64) the
// routing is cheap enough that every workgroup recomputes all of it in LDS
// (top-k, bitmaps, scan, destinations), then copies its own share of the
// rows.  Workgroup 0 also writes the routing outputs.  Each workgroup issues
// the loads of its rows first, so their latency hides behind the routing.
// A block of columns (one 16-byte vector per lane) is shared by `ks`
// workgroups, each storing every ks-th of the k destination rows: at decode
// sizes the column blocks alone would leave a handful of CUs issuing all the
// stores, and routing once more per workgroup costs less than that.
#include "route_common.h"

#include <algorithm>

namespace moe {
namespace {

using namespace route_detail;

constexpr uint32_t kSmallDispatchWorkgroups = 64;

template <int G, int V>
__global__ __launch_bounds__((SingleShape<G>::THREADS)) void route_expand_small_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ dest_of_src, int32_t* __restrict__ src_of_dest,
    const u32x4* __restrict__ x, uint32_t H16, FastDiv div_h16, int ks, u32x4* __restrict__ x_exp) {
    using S = SingleShape<G>;
    __shared__ int32_t ids_lds[kRouteSmallDispatchMaxTokens * kKMax];
    __shared__ unsigned long long masks[kEMax];
    __shared__ int32_t s_cnt[kEMax];
    __shared__ int32_t s_off[kEMax + 1];
    __shared__ int32_t s_dest[kRouteSmallDispatchMaxTokens * kKMax];

    // this workgroup's item of x (one 16-byte vector per lane), loaded first
    const uint32_t n = (uint32_t)T * H16;
    const int js = (int)(blockIdx.x % (uint32_t)ks);  // first of this workgroup's destination slots j
    const uint32_t i = (blockIdx.x / (uint32_t)ks) * S::THREADS + threadIdx.x;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (i < n) v = load_stream(x + i);

    const bool writer = blockIdx.x == 0;
    route_small<G, V>(logits, bias, T, E, k, 1, writer, topk_ids, topk_weights, expert_offsets, expert_counts,
                      ids_lds, masks, s_cnt, s_off);
    const int Epad = (E + 3) & ~3;
    for (int s = threadIdx.x; s < T * k; s += S::THREADS) {
        const int e = ids_lds[s];
        const int d = s_off[e] + slot_rank(masks, Epad, s / k, e);
        s_dest[s] = d;
        if (writer) {
            dest_of_src[s] = d;
            src_of_dest[d] = s;
        }
    }
    __syncthreads();
    if (i < n) {
        const uint32_t t = fastdiv(i, div_h16);
        const uint32_t c = i - t * H16;
        for (int j = js; j < k; j += ks) store_stream(x_exp + (size_t)s_dest[t * k + j] * H16 + c, v);
    }
}

template <int G, int V>
hipError_t launch_gv(const RouteArgs& a, const void* x, int H, void* x_expanded, hipStream_t stream) {
    using S = SingleShape<G>;
    const uint32_t H16 = (uint32_t)H / 8;
    const uint32_t n = (uint32_t)a.T * H16;
    const uint32_t blocks = n == 0 ? 1 : (n + S::THREADS - 1) / S::THREADS;
    // split the k destination rows until about kSmallDispatchWorkgroups workgroups store
    const uint32_t want = (kSmallDispatchWorkgroups + blocks - 1) / blocks;
    const int ks = (int)std::min<uint32_t>((uint32_t)a.k, std::max<uint32_t>(1u, want));
    route_expand_small_kernel<G, V><<<blocks * ks, S::THREADS, 0, stream>>>(
        a.logits, a.bias, a.T, a.E, a.k, a.topk_ids, a.topk_weights, a.expert_offsets, a.expert_counts,
        a.dest_of_src, a.src_of_dest, static_cast<const u32x4*>(x), H16, make_fastdiv(H16), ks,
        static_cast<u32x4*>(x_expanded));
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_expand_small(const RouteArgs& a, const void* x, int H, void* x_expanded,
                                     hipStream_t stream) {
    switch (route_lanes_per_token(a.E) * 16 + route_keys_per_lane(a.E)) {
        case 1 * 16 + 4: return launch_gv<1, 4>(a, x, H, x_expanded, stream);
        case 2 * 16 + 4: return launch_gv<2, 4>(a, x, H, x_expanded, stream);
        case 4 * 16 + 4: return launch_gv<4, 4>(a, x, H, x_expanded, stream);
        case 8 * 16 + 4: return launch_gv<8, 4>(a, x, H, x_expanded, stream);
        case 8 * 16 + 8: return launch_gv<8, 8>(a, x, H, x_expanded, stream);
        case 16 * 16 + 8: return launch_gv<16, 8>(a, x, H, x_expanded, stream);
        case 32 * 16 + 8: return launch_gv<32, 8>(a, x, H, x_expanded, stream);
        default: return launch_gv<64, 8>(a, x, H, x_expanded, stream);
    }
}

}  // namespace moe
