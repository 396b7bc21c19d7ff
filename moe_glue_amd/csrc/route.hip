// moe_route on gfx950: softmax top-k, expert histogram, prefix-sum offsets and
// the stable permutation maps.
//
// "CuTeDSL at Perplexity", MoE dispatch/combine > Local, describes two shapes
// of the dispatch's routing step: for few tokens one block reads all the
// routing information; for many tokens the routing is split over many blocks,
// indices are first assigned per block and then combined across blocks through
// global memory.  Both exist here:
//
//   single workgroup (T <= 256): top-k, histogram, scan and maps in one launch;
//   multi workgroup: kernel 1 (one workgroup per 64 tokens) does top-k, the
//     block-local histogram and each slot's rank inside the block; kernel 2
//     sums the per-block histograms (column prefix over blocks + totals),
//     scans the totals into offsets in LDS and writes the final maps.
//
// The page's blocks claim slots with shared-memory atomic increments, which
// gives each expert's list in arbitrary order.  Here the order is fixed
// (ascending token inside each expert): each 64-token chunk builds, per
// expert, a 64-bit bitmap of the tokens that picked it (LDS atomic OR, which
// commutes), and a slot's rank is the popcount of the bits below its token.
//
// Top-k: G lanes cooperate on one token (4 keys per lane, 8 above 256
// experts).  Each of the k rounds takes the per-lane maximum of a 64-bit key
// (orderable fp32 key in the high word, ~expert in the low word, so equal
// keys prefer the lower expert) and a butterfly over the G lanes with
// ds_swizzle (xor < 32) and ds_bpermute (xor 32).
#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kChunk = 64;     // tokens per rank bitmap
constexpr int kKMax = 16;
constexpr int kEMax = 512;
constexpr int kMaxChunks = kRouteFusedMaxTokens / kChunk;

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));

// fp32 -> uint32 whose unsigned order is the float order, with -0 == +0.
__device__ __forceinline__ uint32_t orderable(float f) {
    uint32_t u = __builtin_bit_cast(uint32_t, f);
    if ((u & 0x7FFFFFFFu) == 0) u = 0;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float unorderable(uint32_t o) {
    uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
    return __builtin_bit_cast(float, u);
}

template <int MASK>
__device__ __forceinline__ uint32_t lane_xor(uint32_t v) {
    if constexpr (MASK < 32) {
        // ds_swizzle bit mode: and_mask = 0x1f, or_mask = 0, xor_mask = MASK
        return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1f | (MASK << 10));
    } else {
        return (uint32_t)__shfl_xor((int)v, MASK);
    }
}

template <int MASK>
__device__ __forceinline__ uint64_t max_with_lane(uint64_t v) {
    uint32_t lo = lane_xor<MASK>((uint32_t)v);
    uint32_t hi = lane_xor<MASK>((uint32_t)(v >> 32));
    uint64_t o = ((uint64_t)hi << 32) | lo;
    return o > v ? o : v;
}

// Maximum over each aligned group of G lanes (all lanes of the wave active).
template <int G>
__device__ __forceinline__ uint64_t group_max(uint64_t v) {
    if constexpr (G > 1) v = max_with_lane<1>(v);
    if constexpr (G > 2) v = max_with_lane<2>(v);
    if constexpr (G > 4) v = max_with_lane<4>(v);
    if constexpr (G > 8) v = max_with_lane<8>(v);
    if constexpr (G > 16) v = max_with_lane<16>(v);
    if constexpr (G > 32) v = max_with_lane<32>(v);
    return v;
}

// Launch shape per lanes-per-token G and keys-per-lane V: P passes of
// THREADS/G tokens cover one 64-token chunk.  THREADS is at most 512, or
// 1024 when that keeps the P*V logits each lane preloads within 32 registers.
template <int G, int V>
struct Shape {
    static constexpr int P0 = (kChunk * G / 512) > 1 ? (kChunk * G / 512) : 1;
    static constexpr int P = (P0 * V > 32) ? (32 / V) : P0;
    static constexpr int THREADS = kChunk * G / P;
    static constexpr int TOK_PER_PASS = THREADS / G;
    static_assert(P * TOK_PER_PASS == kChunk, "one chunk per P passes");
};

// Top-k of the 64 tokens [tok0, tok0 + 64) of which those below T exist.
// Writes topk_ids / topk_weights to global memory and the ids to ids_lds
// ([64][k], token-major).  Every lane of the workgroup must call this.
template <int G, int V>
__device__ __forceinline__ void topk_chunk(const float* __restrict__ logits, const float* __restrict__ bias, int T,
                                           int E, int k, int tok0, int32_t* __restrict__ topk_ids,
                                           float* __restrict__ topk_weights, int32_t* ids_lds) {
    using S = Shape<G, V>;
    const int grp = threadIdx.x / G;
    const int gl = threadIdx.x % G;

    // all loads of the chunk first, so their latencies overlap
    float vals[S::P][V];
#pragma unroll
    for (int p = 0; p < S::P; ++p) {
        const int t = tok0 + p * S::TOK_PER_PASS + grp;
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int e = gl + G * i;
            vals[p][i] = (t < T && e < E) ? logits[(size_t)t * E + e] : 0.0f;
        }
    }
    float bv[V];
#pragma unroll
    for (int i = 0; i < V; ++i) {
        const int e = gl + G * i;
        bv[i] = (bias != nullptr && e < E) ? bias[e] : 0.0f;
    }

#pragma unroll
    for (int p = 0; p < S::P; ++p) {
        const int tl = p * S::TOK_PER_PASS + grp;
        const int t = tok0 + tl;
        const bool live = t < T;
        uint64_t key[V];
#pragma unroll
        for (int i = 0; i < V; ++i) {
            const int e = gl + G * i;
            float kf = vals[p][i];
            if (bias != nullptr) kf = kf + bv[i];
            key[i] = (live && e < E) ? (((uint64_t)orderable(kf) << 32) | (uint32_t)~(uint32_t)e) : 0ull;
        }
        uint32_t wid[kKMax];
        float wkey[kKMax];
#pragma unroll
        for (int r = 0; r < kKMax; ++r) {
            if (r < k) {  // k is uniform: no divergence around the lane exchange
                uint64_t best = key[0];
#pragma unroll
                for (int i = 1; i < V; ++i) best = key[i] > best ? key[i] : best;
                const uint64_t win = group_max<G>(best);
#pragma unroll
                for (int i = 0; i < V; ++i)
                    if (key[i] == win) key[i] = 0ull;
                wid[r] = ~(uint32_t)win;
                wkey[r] = unorderable((uint32_t)(win >> 32));
            }
        }
        if (live) {
            float denom = 0.0f;
#pragma unroll
            for (int r = 0; r < kKMax; ++r)
                if (r < k) denom += expf(wkey[r] - wkey[0]);
#pragma unroll
            for (int r = 0; r < kKMax; ++r) {
                if (r < k && (r % G) == gl) {
                    const size_t s = (size_t)t * k + r;
                    topk_ids[s] = (int32_t)wid[r];
                    topk_weights[s] = expf(wkey[r] - wkey[0]) / denom;
                    ids_lds[tl * k + r] = (int32_t)wid[r];
                }
            }
        }
    }
}

// Per-expert token bitmaps of `ntok` tokens (ids in ids_lds, token-major [ntok][k]):
// masks[c * Epad + e] bit b set <=> token c*64 + b picked expert e.
template <int THREADS>
__device__ __forceinline__ void build_masks(const int32_t* ids_lds, int ntok, int k, int Epad, int nchunks,
                                            unsigned long long* masks) {
    for (int i = threadIdx.x; i < nchunks * Epad; i += THREADS) masks[i] = 0ull;
    __syncthreads();
    for (int s = threadIdx.x; s < ntok * k; s += THREADS) {
        const int tl = s / k;
        const int e = ids_lds[s];
        atomicOr(&masks[(tl >> 6) * Epad + e], 1ull << (tl & 63));
    }
    __syncthreads();
}

// Rank of token tl among the block's tokens that picked expert e.
__device__ __forceinline__ int slot_rank(const unsigned long long* masks, int Epad, int tl, int e) {
    const int c = tl >> 6;
    const unsigned long long below = (1ull << (tl & 63)) - 1ull;
    int r = __popcll(masks[c * Epad + e] & below);
    for (int c2 = 0; c2 < c; ++c2) r += __popcll(masks[c2 * Epad + e]);
    return r;
}

__device__ __forceinline__ int mask_count(const unsigned long long* masks, int Epad, int nchunks, int e) {
    int n = 0;
    for (int c = 0; c < nchunks; ++c) n += __popcll(masks[c * Epad + e]);
    return n;
}

// Exclusive prefix sum of in[0..n) into out[0..n], out[n] = total; n <= 512.
// Run by wave 0 only: each lane owns ceil(n/64) consecutive entries.
__device__ __forceinline__ void wave0_exclusive_scan(const int32_t* in, int32_t* out, int n) {
    if (threadIdx.x >= kWave) return;
    const int lane = threadIdx.x;
    const int per = (n + kWave - 1) / kWave;
    const int base = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
        if (base + i < n) local += in[base + i];
    int incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int y = __shfl_up(incl, d);
        if (lane >= d) incl += y;
    }
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
        if (base + i < n) {
            out[base + i] = run;
            run += in[base + i];
        }
    }
    if (lane == kWave - 1) out[n] = incl;
}

// ------------------------------------------------------------ single workgroup
template <int G, int V>
__global__ __launch_bounds__((Shape<G, V>::THREADS)) void route_single_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ dest_of_src, int32_t* __restrict__ src_of_dest) {
    constexpr int THREADS = Shape<G, V>::THREADS;
    __shared__ int32_t ids_lds[kRouteFusedMaxTokens * kKMax];
    __shared__ unsigned long long masks[kMaxChunks * kEMax];
    __shared__ int32_t s_cnt[kEMax];
    __shared__ int32_t s_off[kEMax + 1];

    const int Epad = (E + 3) & ~3;
    const int nchunks = (T + kChunk - 1) / kChunk;
    for (int c = 0; c < nchunks; ++c)
        topk_chunk<G, V>(logits, bias, T, E, k, c * kChunk, topk_ids, topk_weights, ids_lds + c * kChunk * k);
    __syncthreads();
    build_masks<THREADS>(ids_lds, T, k, Epad, nchunks, masks);
    for (int e = threadIdx.x; e < E; e += THREADS) s_cnt[e] = mask_count(masks, Epad, nchunks, e);
    __syncthreads();
    wave0_exclusive_scan(s_cnt, s_off, E);
    __syncthreads();
    for (int e = threadIdx.x; e <= E; e += THREADS) expert_offsets[e] = s_off[e];
    if (expert_counts != nullptr)
        for (int e = threadIdx.x; e < E; e += THREADS) expert_counts[e] = s_cnt[e];
    for (int s = threadIdx.x; s < T * k; s += THREADS) {
        const int e = ids_lds[s];
        const int d = s_off[e] + slot_rank(masks, Epad, s / k, e);
        dest_of_src[s] = d;
        src_of_dest[d] = s;
    }
}

// ------------------------------------------------------------- multi workgroup
// Kernel 1: workgroup b owns tokens [64b, 64b + 64).  Writes top-k, each
// slot's rank inside the workgroup (into dest_of_src, finished by kernel 2)
// and the workgroup's histogram (workspace row b, Epad ints, zero padded).
template <int G, int V>
__global__ __launch_bounds__((Shape<G, V>::THREADS)) void route_multi_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int32_t* __restrict__ dest_of_src,
    int32_t* __restrict__ block_counts) {
    constexpr int THREADS = Shape<G, V>::THREADS;
    __shared__ int32_t ids_lds[kChunk * kKMax];
    __shared__ unsigned long long masks[kEMax];

    const int Epad = (E + 3) & ~3;
    const int tok0 = blockIdx.x * kChunk;
    const int ntok = min(kChunk, T - tok0);
    topk_chunk<G, V>(logits, bias, T, E, k, tok0, topk_ids, topk_weights, ids_lds);
    __syncthreads();
    build_masks<THREADS>(ids_lds, ntok, k, Epad, 1, masks);
    for (int s = threadIdx.x; s < ntok * k; s += THREADS)
        dest_of_src[(size_t)tok0 * k + s] = slot_rank(masks, Epad, s / k, ids_lds[s]);
    for (int e = threadIdx.x; e < Epad; e += THREADS)
        block_counts[(size_t)blockIdx.x * Epad + e] = (e < E) ? __popcll(masks[e]) : 0;
}

// Kernel 2: every workgroup sums the histogram rows of all workgroups (one
// int4 of experts per lane, rows spread over the lanes) into totals and into
// the prefix over workgroups before it, scans the totals into offsets, and
// finishes its own slots: dest = offset[e] + prefix[e] + rank.
constexpr int kPlaceThreads = 512;

__global__ __launch_bounds__(kPlaceThreads) void route_multi_place_kernel(
    const int32_t* __restrict__ block_counts, int nb, int T, int E, int k, const int32_t* __restrict__ topk_ids,
    int32_t* __restrict__ dest_of_src, int32_t* __restrict__ src_of_dest, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_counts) {
    __shared__ i32x4 part_tot[kPlaceThreads];
    __shared__ i32x4 part_pre[kPlaceThreads];
    __shared__ int32_t s_tot[kEMax];
    __shared__ int32_t s_pre[kEMax];
    __shared__ int32_t s_off[kEMax + 1];

    const int Epad = (E + 3) & ~3;
    const int Q = Epad / 4;              // int4 per histogram row (<= 128)
    const int RP = kPlaceThreads / Q;    // rows read in parallel
    const int b = blockIdx.x;
    const int q = threadIdx.x % Q;
    const int rg = threadIdx.x / Q;

    i32x4 tot = {0, 0, 0, 0};
    i32x4 pre = {0, 0, 0, 0};
    if (rg < RP) {
        const i32x4* rows = reinterpret_cast<const i32x4*>(block_counts);
#pragma unroll 4
        for (int row = rg; row < nb; row += RP) {
            const i32x4 c = rows[(size_t)row * Q + q];
            tot += c;
            if (row < b) pre += c;
        }
    }
    part_tot[threadIdx.x] = tot;
    part_pre[threadIdx.x] = pre;
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += kPlaceThreads) {
        const int qe = e >> 2, ce = e & 3;
        int st = 0, sp = 0;
        for (int g = 0; g < RP; ++g) {
            st += part_tot[g * Q + qe][ce];
            sp += part_pre[g * Q + qe][ce];
        }
        s_tot[e] = st;
        s_pre[e] = sp;
    }
    __syncthreads();
    wave0_exclusive_scan(s_tot, s_off, E);
    __syncthreads();
    if (b == 0) {
        for (int e = threadIdx.x; e <= E; e += kPlaceThreads) expert_offsets[e] = s_off[e];
        if (expert_counts != nullptr)
            for (int e = threadIdx.x; e < E; e += kPlaceThreads) expert_counts[e] = s_tot[e];
    }
    const int tok0 = b * kChunk;
    const int ntok = min(kChunk, T - tok0);
    for (int s = threadIdx.x; s < ntok * k; s += kPlaceThreads) {
        const size_t gs = (size_t)tok0 * k + s;
        const int e = topk_ids[gs];
        const int d = s_off[e] + s_pre[e] + dest_of_src[gs];
        dest_of_src[gs] = d;
        src_of_dest[d] = (int32_t)gs;
    }
}

template <int G, int V>
hipError_t launch_route_gv(const RouteArgs& a, RouteVariant v, hipStream_t stream) {
    constexpr int THREADS = Shape<G, V>::THREADS;
    if (v == RouteVariant::SingleWorkgroup) {
        route_single_kernel<G, V><<<1, THREADS, 0, stream>>>(a.logits, a.bias, a.T, a.E, a.k, a.topk_ids,
                                                             a.topk_weights, a.expert_offsets, a.expert_counts,
                                                             a.dest_of_src, a.src_of_dest);
        return hipGetLastError();
    }
    const int nb = route_num_blocks(a.T);
    int32_t* counts = static_cast<int32_t*>(a.workspace);
    route_multi_topk_kernel<G, V><<<nb, THREADS, 0, stream>>>(a.logits, a.bias, a.T, a.E, a.k, a.topk_ids,
                                                              a.topk_weights, a.dest_of_src, counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    route_multi_place_kernel<<<nb, kPlaceThreads, 0, stream>>>(counts, nb, a.T, a.E, a.k, a.topk_ids, a.dest_of_src,
                                                               a.src_of_dest, a.expert_offsets, a.expert_counts);
    return hipGetLastError();
}

}  // namespace

int route_lanes_per_token(int E) {
    const int need = (E + 3) / 4;
    int G = 1;
    while (G < need && G < 64) G <<= 1;
    return G;
}

RouteVariant route_pick_variant(int T, RouteVariant requested) {
    if (T <= 0) return RouteVariant::SingleWorkgroup;  // writes the all-zero offsets
    if (requested == RouteVariant::SingleWorkgroup && T <= kRouteFusedMaxTokens) return requested;
    if (requested == RouteVariant::MultiWorkgroup) return requested;
    return T <= kChunk ? RouteVariant::SingleWorkgroup : RouteVariant::MultiWorkgroup;
}

hipError_t launch_route(const RouteArgs& a, RouteVariant variant, hipStream_t stream) {
    const RouteVariant v = route_pick_variant(a.T, variant);
    if (a.E > 256) return launch_route_gv<64, 8>(a, v, stream);
    switch (route_lanes_per_token(a.E)) {
        case 1: return launch_route_gv<1, 4>(a, v, stream);
        case 2: return launch_route_gv<2, 4>(a, v, stream);
        case 4: return launch_route_gv<4, 4>(a, v, stream);
        case 8: return launch_route_gv<8, 4>(a, v, stream);
        case 16: return launch_route_gv<16, 4>(a, v, stream);
        case 32: return launch_route_gv<32, 4>(a, v, stream);
        default: return launch_route_gv<64, 4>(a, v, stream);
    }
}

}  // namespace moe
