// Device-side building blocks of the routing kernels (moe_route and the
// fused small-batch route+expand): order-preserving keys, DPP/permlane group
// reductions, the per-token top-k, the per-expert token bitmaps that give
// each slot its stable rank, and the LDS exclusive scan.  See route.hip for
// how they are put together.
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace moe {
namespace route_detail {

constexpr int kChunk = 64;  // tokens per rank bitmap
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

// Top-k of token t by the G lanes of one group (lane gl of the group).
// Every lane of the wave must call this (the reductions cross lanes); lanes
// with t >= T compute on empty keys and write nothing.  Writes the ids to
// ids_lds[tl * k + r], and topk_ids / topk_weights unless topk_ids is null.
template <int G, int V>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, const float* __restrict__ bias, int T,
                                           int E, int k, int t, int tl, int gl, int32_t* __restrict__ topk_ids,
                                           float* __restrict__ topk_weights, int32_t* ids_lds) {
    static_assert(V > 0 && (V & (V - 1)) == 0, "the tournament pairs keys: V must be a power of two");
    constexpr int NJ = (kKMax + G - 1) / G;  // slots a lane may own: r = gl + G*j
    const bool live = t < T;
    // loads from clamped addresses, all issued before any is used (a load
    // under a lane condition would make the compiler wait for it on the spot);
    // the caller guarantees T >= 1
    const size_t row = (size_t)min(t, T - 1) * E;
    float vals[V];
#pragma unroll
    for (int i = 0; i < V; ++i) vals[i] = logits[row + min(gl + G * i, E - 1)];
    if (bias != nullptr) {  // uniform
        float b[V];
#pragma unroll
        for (int i = 0; i < V; ++i) b[i] = bias[min(gl + G * i, E - 1)];
#pragma unroll
        for (int i = 0; i < V; ++i) vals[i] = vals[i] + b[i];
    }
    // key[i] of expert gl + G*i: orderable fp32 key, 0 = absent or taken
    // (every real key is above 0: orderable(-inf) = 0x007FFFFF)
    uint32_t key[V];
#pragma unroll
    for (int i = 0; i < V; ++i) key[i] = (live && gl + G * i < E) ? orderable(vals[i]) : 0u;
    uint32_t my_id[NJ];
    uint32_t my_key[NJ];
    uint32_t top0 = 0;
    // rounds as a rolled loop: the small-batch kernels run this code once per
    // workgroup, where fetching an unrolled copy costs more than the loop
#pragma unroll 1
    for (int r = 0; r < k; ++r) {
        {  // k is uniform: no divergence around the lane exchange
            // the lane's best: largest key, lowest expert on equal keys, by a
            // pairwise tournament (log2 V dependent steps, not V - 1): the
            // left candidate holds the lower experts, so it keeps ties
            uint32_t tk[V];
            int ti[V];
#pragma unroll
            for (int i = 0; i < V; ++i) {
                tk[i] = key[i];
                ti[i] = i;
            }
#pragma unroll
            for (int w = 1; w < V; w *= 2)
#pragma unroll
                for (int i = 0; i + w < V; i += 2 * w)
                    if (tk[i + w] > tk[i]) {
                        tk[i] = tk[i + w];
                        ti[i] = ti[i + w];
                    }
            const uint32_t best = tk[0];
            const int bi = ti[0];
            // the group's best key, then the lowest expert holding it
            const uint32_t top = group_reduce<G, Op::Max>(best);
            const uint32_t mine = (best == top) ? (uint32_t)(gl + G * bi) : 0xFFFFFFFFu;
            const uint32_t win = group_reduce<G, Op::Min>(mine);
#pragma unroll
            for (int i = 0; i < V; ++i)  // the owner retires the winner
                if ((uint32_t)(gl + G * i) == win) key[i] = 0u;
            if (r == 0) top0 = top;
#pragma unroll
            for (int j = 0; j < NJ; ++j)  // static indices: r = gl + G*j
                if (r == gl + G * j) {
                    my_id[j] = win;
                    my_key[j] = top;
                }
        }
    }
    // weights: softmax over the k selected keys, relative to the largest
    const float key0 = unorderable(top0);
    float ex[NJ];
    float part = 0.0f;
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int r = gl + G * j;
        ex[j] = (r < k) ? expf(unorderable(my_key[j]) - key0) : 0.0f;
        part += ex[j];
    }
    const float denom = __builtin_bit_cast(float, group_reduce<G, Op::FAdd>(__builtin_bit_cast(uint32_t, part)));
    if (live) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int r = gl + G * j;
            if (r < k) {
                if (topk_ids != nullptr) {
                    const size_t s = (size_t)t * k + r;
                    topk_ids[s] = (int32_t)my_id[j];
                    topk_weights[s] = ex[j] / denom;
                }
                ids_lds[tl * k + r] = (int32_t)my_id[j];
            }
        }
    }
}

// Per-expert token bitmaps: masks[c * Epad + e] bit b set <=> token c*64 + b
// picked expert e.  clear_masks zeroes them (and the per-expert counts, when
// given); callers run it before the top-k, so the barrier that follows the
// top-k orders the clearing before mark_masks.  mark_masks sets each slot's
// bit with an LDS atomic OR (order-free) and counts it, then waits for the
// workgroup.
template <int THREADS>
__device__ __forceinline__ void clear_masks(unsigned long long* masks, int n, int32_t* s_cnt, int E) {
    for (int i = threadIdx.x; i < n; i += THREADS) masks[i] = 0ull;
    if (s_cnt != nullptr)
        for (int e = threadIdx.x; e < E; e += THREADS) s_cnt[e] = 0;
}

template <int THREADS>
__device__ __forceinline__ void mark_masks(const int32_t* ids_lds, int ntok, int k, int Epad,
                                           unsigned long long* masks, int32_t* s_cnt) {
    for (int s = threadIdx.x; s < ntok * k; s += THREADS) {
        const int tl = s / k;
        const int e = ids_lds[s];
        atomicOr(&masks[(tl >> 6) * Epad + e], 1ull << (tl & 63));
        if (s_cnt != nullptr) atomicAdd(&s_cnt[e], 1);
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

// Segment length of an expert with `count` rows: count rounded up to a
// multiple of pad (pad = 1: unpadded).
__device__ __forceinline__ int padded_len(int count, int pad) { return pad == 1 ? count : (count + pad - 1) / pad * pad; }

// Exclusive prefix sum of the padded lengths of in[0..n) (plus add[i] when
// given) into out[0..n], out[n] = total; n <= 512.  Run by wave `w` of the
// workgroup only: each lane owns ceil(n/64) consecutive entries.
__device__ __forceinline__ void wave_exclusive_scan(const int32_t* in, int32_t* out, int n, int pad, int w,
                                                    const int32_t* add = nullptr) {
    if ((int)(threadIdx.x / kWave) != w) return;
    const int lane = threadIdx.x % kWave;
    const int per = (n + kWave - 1) / kWave;
    const int base = lane * per;
    int local = 0;
    for (int i = 0; i < per; ++i)
        if (base + i < n) local += padded_len(in[base + i] + (add ? add[base + i] : 0), pad);
    const int incl = wave_inclusive_sum(local);
    int run = incl - local;
    for (int i = 0; i < per; ++i) {
        if (base + i < n) {
            out[base + i] = run;
            run += padded_len(in[base + i] + (add ? add[base + i] : 0), pad);
        }
    }
    if (lane == kWave - 1) out[n] = incl;
}

__device__ __forceinline__ void wave0_exclusive_scan(const int32_t* in, int32_t* out, int n, int pad) {
    wave_exclusive_scan(in, out, n, pad, 0);
}

// Padding rows of the padded layout get src_of_dest = -1: rows
// [off[e] + cnt[e], off[e+1]) of every expert e.  Experts are dealt to the
// waves of `nblocks` workgroups round-robin; the lanes of a wave stride over
// the expert's padding rows.  No-op when pad == 1.
template <int THREADS>
__device__ __forceinline__ void mark_padding(const int32_t* s_cnt, const int32_t* s_off, int E, int pad, int block,
                                             int nblocks, int32_t* __restrict__ src_of_dest) {
    if (pad == 1) return;
    constexpr int NW = THREADS / kWave;
    const int lane = threadIdx.x % kWave;
    const int w = threadIdx.x / kWave;
    for (int e = block * NW + w; e < E; e += nblocks * NW) {
        const int first = s_off[e] + s_cnt[e];
        const int last = s_off[e + 1];
        for (int p = first + lane; p < last; p += kWave) src_of_dest[p] = -1;
    }
}

// Sum of v over the lanes of the wave that sit a multiple of QP apart (QP a
// power of two <= 32): DPP rotations inside each 16-lane row, then the
// permlane swaps across rows.
template <int QP>
__device__ __forceinline__ uint32_t add_lanes(uint32_t v) {
    if constexpr (QP <= 1) v += dpp<0x121>(v);  // row_ror:1
    if constexpr (QP <= 2) v += dpp<0x122>(v);  // row_ror:2
    if constexpr (QP <= 4) v += dpp<0x124>(v);  // row_ror:4
    if constexpr (QP <= 8) v += dpp<0x128>(v);  // row_ror:8
    if constexpr (QP <= 16) {
        const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        v = p[0] + p[1];
    }
    const auto p = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return p[0] + p[1];
}

// Launch shapes.
// Multi-workgroup top-k: one token per group of G lanes, one pass, TOK tokens
// per workgroup: 16 (THREADS = 16*G = 64..1024) for G >= 4, one wave below.
template <int G>
struct TopkShape {
    static constexpr int TOK = (G >= 4) ? 16 : kWave / G;
    static constexpr int THREADS = TOK * G;
};
// Single workgroup: up to 1024 lanes, at most 64 tokens per pass.
template <int G>
struct SingleShape {
    static constexpr int THREADS = (kChunk * G < 1024) ? kChunk * G : 1024;
    static constexpr int TOK_PER_PASS = THREADS / G;
};


// Top-k, histogram, offsets (segments padded to a multiple of `pad`) and
// ranks of T <= kRouteFusedMaxTokens tokens by one workgroup, all in LDS:
// ids_lds [T][k], masks [nchunks][Epad], s_cnt [E], s_off [E+1].  Waves whose tokens all lie at or past T skip the
// top-k.  When `write` is set the workgroup also writes topk_ids,
// topk_weights, expert_offsets and expert_counts (not the maps).
template <int G, int V>
__device__ __forceinline__ void route_small(const float* __restrict__ logits, const float* __restrict__ bias, int T,
                                            int E, int k, int pad, bool write, int32_t* __restrict__ topk_ids,
                                            float* __restrict__ topk_weights, int32_t* __restrict__ expert_offsets,
                                            int32_t* __restrict__ expert_counts, int32_t* ids_lds,
                                            unsigned long long* masks, int32_t* s_cnt, int32_t* s_off) {
    using S = SingleShape<G>;
    const int Epad = (E + 3) & ~3;
    const int grp = threadIdx.x / G;
    const int gl = threadIdx.x % G;
    const int wave_first = (threadIdx.x / kWave) * (kWave / G);  // first token slot of this wave in a pass
    const int nchunks = (T + kChunk - 1) / kChunk;
    clear_masks<S::THREADS>(masks, nchunks * Epad, s_cnt, E);
    for (int t0 = 0; t0 < T; t0 += S::TOK_PER_PASS) {
        if (t0 + wave_first < T)  // wave-uniform: the lane exchange stays whole-wave
            topk_token<G, V>(logits, bias, T, E, k, t0 + grp, t0 + grp, gl, write ? topk_ids : nullptr,
                             topk_weights, ids_lds);
    }
    __syncthreads();
    mark_masks<S::THREADS>(ids_lds, T, k, Epad, masks, s_cnt);
    wave0_exclusive_scan(s_cnt, s_off, E, pad);
    __syncthreads();
    if (write) {
        for (int e = threadIdx.x; e <= E; e += S::THREADS) expert_offsets[e] = s_off[e];
        if (expert_counts != nullptr)
            for (int e = threadIdx.x; e < E; e += S::THREADS) expert_counts[e] = s_cnt[e];
    }
}

}  // namespace route_detail
}  // namespace moe
