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
// stores, and routing once more per workgroup costs less than that.  The same
// kernel serves the padded layout (pad_to) and the FP8 and MXFP8 quantising
// copies.
#include "fp8_common.h"
#include "place_copy.h"
#include "route_common.h"

#include <algorithm>

namespace moe {
namespace {

using namespace route_detail;

constexpr uint32_t kSmallDispatchWorkgroups = 64;

template <int G, int V, int MODE>
__global__ __launch_bounds__((SingleShape<G>::THREADS)) void route_expand_small_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k, int pad,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ dest_of_src, int32_t* __restrict__ src_of_dest,
    const u32x4* __restrict__ x, uint32_t H16, FastDiv div_h16, int ks, void* __restrict__ out,
    void* __restrict__ scales, uint32_t G_groups, int gl, bool mx) {
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
    route_small<G, V>(logits, bias, T, E, k, pad, writer, topk_ids, topk_weights, expert_offsets, expert_counts,
                      ids_lds, masks, s_cnt, s_off);
    mark_padding<S::THREADS>(s_cnt, s_off, E, pad, blockIdx.x, gridDim.x, src_of_dest);  // experts dealt out
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
    if constexpr (MODE == kCopyBf16) {
        if (i < n) {
            const uint32_t t = fastdiv(i, div_h16);
            const uint32_t c = i - t * H16;
            u32x4* x_exp = static_cast<u32x4*>(out);
            for (int j = js; j < k; j += ks) store_stream(x_exp + (size_t)s_dest[t * k + j] * H16 + c, v);
        }
    } else {
        // E4M3 as moe_expand_rows_fp8 (or, with mx, moe_expand_rows_mxfp8): a
        // scale group is gl consecutive lanes of one row (H/8 is a multiple of
        // gl, so no group straddles the end of x)
        float f[8];
        unpack8(v, f);
        const uint32_t amax_bits = group_abs_max(abs_max_bits8(f), gl);
        if (i < n) {
            const uint32_t t = fastdiv(i, div_h16);
            const uint32_t c = i - t * H16;
            const BlockScale bs = block_scale(amax_bits, mx);
            const u32x2 codes = quantize8_e4m3(f, bs.inv, bs.pre);
            const bool first_of_group = (threadIdx.x % (uint32_t)gl) == 0;
            u32x2* q_out = static_cast<u32x2*>(out);
            for (int j = js; j < k; j += ks) {
                const size_t d = (size_t)s_dest[t * k + j];
                __builtin_nontemporal_store(codes, q_out + d * H16 + c);
                if (first_of_group) store_block_scale(scales, d * G_groups + c / (uint32_t)gl, bs, mx);
            }
        }
    }
}

template <int G, int V>
hipError_t launch_gv(const RouteArgs& a, hipStream_t stream) {
    using S = SingleShape<G>;
    const uint32_t H16 = (uint32_t)a.copy_H / 8;
    const uint32_t n = (uint32_t)a.T * H16;
    const uint32_t blocks = n == 0 ? 1 : (n + S::THREADS - 1) / S::THREADS;
    // split the k destination rows until about kSmallDispatchWorkgroups workgroups store
    const uint32_t want = (kSmallDispatchWorkgroups + blocks - 1) / blocks;
    const int ks = (int)std::min<uint32_t>((uint32_t)a.k, std::max<uint32_t>(1u, want));
    const u32x4* x = static_cast<const u32x4*>(a.copy_x);
    if (a.copy_group > 0)
        route_expand_small_kernel<G, V, kCopyFp8><<<blocks * ks, S::THREADS, 0, stream>>>(
            a.logits, a.bias, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.topk_weights, a.expert_offsets, a.expert_counts,
            a.dest_of_src, a.src_of_dest, x, H16, make_fastdiv(H16), ks, a.copy_out, a.copy_scales,
            (uint32_t)(a.copy_H / a.copy_group), a.copy_group / 8, a.copy_mx);
    else
        route_expand_small_kernel<G, V, kCopyBf16><<<blocks * ks, S::THREADS, 0, stream>>>(
            a.logits, a.bias, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.topk_weights, a.expert_offsets, a.expert_counts,
            a.dest_of_src, a.src_of_dest, x, H16, make_fastdiv(H16), ks, a.copy_out, nullptr, 0, 1, false);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route_expand_small(const RouteArgs& a, hipStream_t stream) {
    switch (route_lanes_per_token(a.E) * 16 + route_keys_per_lane(a.E)) {
        case 1 * 16 + 4: return launch_gv<1, 4>(a, stream);
        case 2 * 16 + 4: return launch_gv<2, 4>(a, stream);
        case 4 * 16 + 4: return launch_gv<4, 4>(a, stream);
        case 8 * 16 + 4: return launch_gv<8, 4>(a, stream);
        case 8 * 16 + 8: return launch_gv<8, 8>(a, stream);
        case 16 * 16 + 8: return launch_gv<16, 8>(a, stream);
        case 32 * 16 + 8: return launch_gv<32, 8>(a, stream);
        default: return launch_gv<64, 8>(a, stream);
    }
}

}  // namespace moe
