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
// routing is cheap enough that every workgroup recomputes all of it in LDS,
// then copies its own share of the rows.  Workgroup 0 also writes the routing
// outputs.  Each workgroup issues the loads of its rows first, so their
// latency hides behind the routing.  A block of columns (one 16-byte vector
// per lane) is shared by `ks` workgroups, each storing every ks-th of the k
// destination rows: at decode sizes the column blocks alone would leave a
// handful of CUs issuing all the stores, and routing once more per workgroup
// costs less than that.  The same kernel serves the padded layout (pad_to) and
// the FP8 and MXFP8 quantising copies.
//
// The routing is shaped for latency, since each workgroup runs it once on a
// cold instruction cache and nothing else hides it: the top-k rounds stay a
// rolled loop; each token's picks set its bit in the pick's 64-bit LDS bitmap
// (T <= 64: one word per expert), so counts are popcounts and a slot's rank
// is the popcount of the bits below its token; every wave scans the counts
// itself into its own offset table and every lane forms the destinations of
// its own rows.  Two barriers: after the clearing and after the top-k.  A
// workgroup has as many lanes as one top-k pass over the T tokens needs (G
// per token; 256, 512 or 1024 for the wide expert counts), so no wave idles
// through the top-k: at T = 32, E = 128, 512 lanes took the call from 7.23
// to 6.64 us against 1024 (64 workgroups either way; 128 of 512 lanes,
// one store per lane, 7.1; 32 or 48 workgroups the same as 64).
#include "fp8_common.h"
#include "place_copy.h"
#include "route_common.h"

#include <algorithm>

namespace moe {
namespace {

using namespace route_detail;

constexpr uint32_t kSmallDispatchWorkgroups = 64;
static_assert(kRouteSmallDispatchMaxTokens <= 64, "one bitmap word per expert");

// TH lanes: enough for all T tokens in one top-k pass (G lanes each), so no
// wave idles through the top-k and no more waves than needed are launched.
template <int G, int V, int MODE, int TH>
__global__ __launch_bounds__(TH) void route_expand_small_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k, int pad,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ dest_of_src, int32_t* __restrict__ src_of_dest,
    const u32x4* __restrict__ x, uint32_t H16, FastDiv div_h16, int ks, void* __restrict__ out,
    void* __restrict__ scales, uint32_t G_groups, int gl_q, bool mx) {
    static_assert(TH % kWave == 0 && TH >= G, "whole waves, at least one token per pass");
    constexpr int NW = TH / kWave;
    constexpr int TOK_PER_PASS = TH / G;
    __shared__ int32_t s_ids[kRouteSmallDispatchMaxTokens * kKMax];  // [t][r]: expert of rank r
    __shared__ unsigned long long s_mask[kEMax];                     // bit t: token t picked expert e
    __shared__ int32_t s_off[NW][kEMax + 1];                         // each wave's offset table

    const int lane = (int)(threadIdx.x % kWave);
    const int wave = (int)(threadIdx.x / kWave);

    // this workgroup's item of x (one 16-byte vector per lane), loaded first
    const uint32_t n = (uint32_t)T * H16;
    const int js = (int)(blockIdx.x % (uint32_t)ks);  // first of this workgroup's destination slots j
    const uint32_t i = (blockIdx.x / (uint32_t)ks) * TH + threadIdx.x;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (i < n) v = load_stream(x + i);

    const bool writer = blockIdx.x == 0;
    const int grp = (int)threadIdx.x / G;
    const int gl = (int)threadIdx.x % G;
    const int wave_first = wave * (kWave / G);  // first token slot of this wave in a pass

    for (int e = (int)threadIdx.x; e < E; e += TH) s_mask[e] = 0ull;
    __syncthreads();  // bitmaps clear

    for (int t0 = 0; t0 < T; t0 += TOK_PER_PASS) {
        if (t0 + wave_first >= T) continue;  // wave-uniform: the lane exchange stays whole-wave
        const int t = t0 + grp;
        // ids of token t into s_ids[t][r] (and, from workgroup 0, topk_ids and topk_weights)
        topk_token<G, V>(logits, bias, T, E, k, t, t, gl, writer ? topk_ids : nullptr, topk_weights, s_ids);
        // its picks into the bitmaps: lane gl set ranks gl + G*j (written by this lane)
        if (t < T)
            for (int r = gl; r < k; r += G) atomicOr(&s_mask[s_ids[t * k + r]], 1ull << t);
    }
    __syncthreads();  // every pick in the bitmaps

    // this wave's offset table: exclusive scan of the padded counts (lane
    // owns `per` consecutive experts, their bitmaps read in one go)
    int32_t* off = s_off[wave];
    {
        constexpr int PER_MAX = kEMax / kWave;
        const int per = (E + kWave - 1) / kWave;
        const int base = lane * per;
        const int own = max(0, min(per, E - base));
        int len[PER_MAX];
#pragma unroll
        for (int q = 0; q < PER_MAX; ++q) len[q] = q < own ? __popcll(s_mask[base + q]) : 0;
        if (pad > 1)  // uniform
#pragma unroll
            for (int q = 0; q < PER_MAX; ++q) len[q] = (len[q] + pad - 1) / pad * pad;
        int local = 0;
#pragma unroll
        for (int q = 0; q < PER_MAX; ++q) local += len[q];
        const int incl = wave_inclusive_sum(local);
        int run = incl - local;
#pragma unroll
        for (int q = 0; q < PER_MAX; ++q) {
            if (q < own) off[base + q] = run;
            run += len[q];
        }
        if (lane == kWave - 1) off[E] = incl;
    }
    // destination of slot (t, j): the expert's offset plus the tokens below t that picked it
    auto dest = [&](int t, int j) {
        const int e = s_ids[t * k + j];
        return off[e] + __popcll(s_mask[e] & ((1ull << t) - 1ull));
    };

    if constexpr (MODE == kCopyBf16) {
        if (i < n) {
            const uint32_t t = fastdiv(i, div_h16);
            const uint32_t c = i - t * H16;
            u32x4* x_exp = static_cast<u32x4*>(out);
            for (int j = js; j < k; j += ks) store_stream(x_exp + (size_t)dest((int)t, j) * H16 + c, v);
        }
    } else {
        // E4M3 as moe_expand_rows_fp8 (or, with mx, moe_expand_rows_mxfp8): a
        // scale group is gl_q consecutive lanes of one row (H/8 is a multiple
        // of gl_q, so no group straddles the end of x)
        float f[8];
        unpack8(v, f);
        const uint32_t amax_bits = group_abs_max(abs_max_bits8(f), gl_q);
        if (i < n) {
            const uint32_t t = fastdiv(i, div_h16);
            const uint32_t c = i - t * H16;
            const BlockScale bs = block_scale(amax_bits, mx);
            const u32x2 codes = quantize8_e4m3(f, bs.inv, bs.pre);
            const bool first_of_group = (threadIdx.x % (uint32_t)gl_q) == 0;
            u32x2* q_out = static_cast<u32x2*>(out);
            for (int j = js; j < k; j += ks) {
                const size_t d = (size_t)dest((int)t, j);
                __builtin_nontemporal_store(codes, q_out + d * H16 + c);
                if (first_of_group) store_block_scale(scales, d * G_groups + c / (uint32_t)gl_q, bs, mx);
            }
        }
    }

    // padding rows (src_of_dest = -1): experts dealt to the waves of the grid
    if (pad > 1)
        for (int e = (int)blockIdx.x * NW + wave; e < E; e += (int)gridDim.x * NW)
            for (int p = off[e] + __popcll(s_mask[e]) + lane; p < off[e + 1]; p += kWave) src_of_dest[p] = -1;
    if (writer) {
        for (int e = (int)threadIdx.x; e <= E; e += TH) expert_offsets[e] = off[e];
        if (expert_counts != nullptr)
            for (int e = (int)threadIdx.x; e < E; e += TH) expert_counts[e] = __popcll(s_mask[e]);
        for (int s2 = (int)threadIdx.x; s2 < T * k; s2 += TH) {
            const int d = dest(s2 / k, s2 % k);
            dest_of_src[s2] = d;
            src_of_dest[d] = s2;
        }
    }
}

template <int G, int V, int TH>
hipError_t launch_th(const RouteArgs& a, hipStream_t stream) {
    const uint32_t H16 = (uint32_t)a.copy_H / 8;
    const uint32_t n = (uint32_t)a.T * H16;
    const uint32_t blocks = n == 0 ? 1 : (n + TH - 1) / TH;
    // split the k destination rows until about kSmallDispatchWorkgroups workgroups store
    const uint32_t want = (kSmallDispatchWorkgroups + blocks - 1) / blocks;
    const int ks = (int)std::min<uint32_t>((uint32_t)a.k, std::max<uint32_t>(1u, want));
    const u32x4* x = static_cast<const u32x4*>(a.copy_x);
    if (a.copy_group > 0)
        route_expand_small_kernel<G, V, kCopyFp8, TH><<<blocks * ks, TH, 0, stream>>>(
            a.logits, a.bias, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.topk_weights, a.expert_offsets, a.expert_counts,
            a.dest_of_src, a.src_of_dest, x, H16, make_fastdiv(H16), ks, a.copy_out, a.copy_scales,
            (uint32_t)(a.copy_H / a.copy_group), a.copy_group / 8, a.copy_mx);
    else
        route_expand_small_kernel<G, V, kCopyBf16, TH><<<blocks * ks, TH, 0, stream>>>(
            a.logits, a.bias, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.topk_weights, a.expert_offsets, a.expert_counts,
            a.dest_of_src, a.src_of_dest, x, H16, make_fastdiv(H16), ks, a.copy_out, nullptr, 0, 1, false);
    return hipGetLastError();
}

template <int G, int V>
hipError_t launch_gv(const RouteArgs& a, hipStream_t stream) {
    constexpr int FULL = SingleShape<G>::THREADS;  // lanes for 64 tokens, at most 1024
    if constexpr (FULL == 1024) {
        if (a.T * G <= 256) return launch_th<G, V, 256>(a, stream);
        if (a.T * G <= 512) return launch_th<G, V, 512>(a, stream);
    }
    return launch_th<G, V, FULL>(a, stream);
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
