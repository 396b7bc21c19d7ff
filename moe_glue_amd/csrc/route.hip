// moe_route on gfx950: softmax top-k, expert histogram, prefix-sum offsets and
// the stable permutation maps.
//
// "CuTeDSL at Perplexity", MoE dispatch/combine > Local, describes two shapes
// of the dispatch's routing step: for few tokens one block reads all the
// routing information; for many tokens the routing is split over many blocks,
// indices are first assigned per block and then combined across blocks through
// global memory.  Both exist here:
//
//   single workgroup (small T): top-k, histogram, scan and maps in one launch;
//   multi workgroup:
//     1. top-k     one workgroup per 16 tokens (64 below 4 lanes per token),
//                  so even a few thousand tokens spread over every CU: writes
//                  the top-k, each slot's rank inside the workgroup and the
//                  workgroup's expert histogram (one workspace row);
//     2. scan      one workgroup per 4 experts: exclusive prefix of the
//                  histogram rows down each expert column, plus the totals;
//     3. place     per workgroup of step 1: scan the totals into offsets (in
//                  LDS) and write dest = offset + prefix + rank and its inverse.
//   Each launch costs a few microseconds on its own, so while the histogram
//   matrix is small (up to 128 KiB of count bytes) steps 2 and 3 run as one
//   launch in which every workgroup reads the whole matrix.  For
//   moe_route_expand the place step also writes the row list of the grouped
//   expand (expand.hip).
//
// The page's blocks claim slots with shared-memory atomic increments, which
// gives each expert's list in arbitrary order.  Here the order is fixed
// (ascending token inside each expert): the workgroup builds, per expert, a
// 64-bit bitmap of its tokens that picked it (LDS atomic OR, which commutes),
// and a slot's rank is the popcount of the bits below its token.
//
// Top-k: G lanes cooperate on one token (8 keys per lane above 32 experts,
// else 4).  Each of the k rounds finds the group's largest key (fp32 mapped
// to an order-preserving uint32, -0 folded onto +0) and then the lowest
// expert holding it, with two DPP/permlane reductions over the G lanes; the
// lane that owns the winner retires it.  Each lane then computes only the
// exponentials of the slots it writes, and one more reduction sums them.
#include "fp8_common.h"
#include "place_copy.h"
#include "route_common.h"

#include <algorithm>

namespace moe {
namespace {

using namespace route_detail;

// ------------------------------------------------------------ single workgroup
template <int G, int V>
__global__ __launch_bounds__((SingleShape<G>::THREADS)) void route_single_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k, int pad,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int32_t* __restrict__ expert_offsets,
    int32_t* __restrict__ expert_counts, int32_t* __restrict__ dest_of_src, int32_t* __restrict__ src_of_dest) {
    using S = SingleShape<G>;
    __shared__ int32_t ids_lds[kRouteFusedMaxTokens * kKMax];
    __shared__ unsigned long long masks[kMaxChunks * kEMax];
    __shared__ int32_t s_cnt[kEMax];
    __shared__ int32_t s_off[kEMax + 1];

    route_small<G, V>(logits, bias, T, E, k, pad, true, topk_ids, topk_weights, expert_offsets, expert_counts,
                      ids_lds, masks, s_cnt, s_off);
    const int Epad = (E + 3) & ~3;
    mark_padding<S::THREADS>(s_cnt, s_off, E, pad, 0, 1, src_of_dest);
    for (int s = threadIdx.x; s < T * k; s += S::THREADS) {
        const int e = ids_lds[s];
        const int d = s_off[e] + slot_rank(masks, Epad, s / k, e);
        dest_of_src[s] = d;
        src_of_dest[d] = s;
    }
}

// ------------------------------------------------------------- multi workgroup
// 1. Workgroup b owns tokens [b*TOK, b*TOK + TOK).  Writes the top-k, each
// slot's rank inside the workgroup (into dest_of_src, finished later; not
// with RANKS = false, whose second launch ranks the slots itself) and the
// workgroup's histogram as workspace row b: Epad int32 (three-launch form) or
// one count byte per expert in route_byte_row_vectors(E) 16-byte vectors
// (two-launch form; a count is at most TOK <= 64), zero padded.
template <int G, int V, bool BYTES, bool RANKS = true>
__global__ __launch_bounds__((TopkShape<G>::THREADS)) void route_topk_kernel(
    const float* __restrict__ logits, const float* __restrict__ bias, int T, int E, int k,
    int32_t* __restrict__ topk_ids, float* __restrict__ topk_weights, int32_t* __restrict__ dest_of_src,
    int32_t* __restrict__ block_counts) {
    using S = TopkShape<G>;
    static_assert(S::TOK <= kChunk, "one rank bitmap per workgroup");
    __shared__ int32_t ids_lds[S::TOK * kKMax];
    __shared__ unsigned long long masks[kEMax];

    const int Epad = (E + 3) & ~3;
    const int tok0 = blockIdx.x * S::TOK;
    const int ntok = min(S::TOK, T - tok0);
    const int grp = threadIdx.x / G;
    clear_masks<S::THREADS>(masks, Epad, nullptr, 0);
    topk_token<G, V>(logits, bias, T, E, k, tok0 + grp, grp, threadIdx.x % G, topk_ids, topk_weights, ids_lds);
    __syncthreads();
    mark_masks<S::THREADS>(ids_lds, ntok, k, Epad, masks, nullptr);
    if constexpr (RANKS)
        for (int s = threadIdx.x; s < ntok * k; s += S::THREADS)
            dest_of_src[(size_t)tok0 * k + s] = slot_rank(masks, Epad, s / k, ids_lds[s]);
    if constexpr (BYTES) {
        const int words = route_byte_row_vectors(E) * 4;  // 4 experts per word
        for (int i = threadIdx.x; i < words; i += S::THREADS) {
            uint32_t w = 0;
#pragma unroll
            for (int b = 0; b < 4; ++b)
                if (4 * i + b < E) w |= (uint32_t)__popcll(masks[4 * i + b]) << (8 * b);
            block_counts[(size_t)blockIdx.x * words + i] = (int32_t)w;
        }
    } else {
        for (int e = threadIdx.x; e < Epad; e += S::THREADS)
            block_counts[(size_t)blockIdx.x * Epad + e] = (e < E) ? __popcll(masks[e]) : 0;
    }
}

// Exclusive scan of one int4 per lane over a workgroup of THREADS lanes.
template <int THREADS>
__device__ __forceinline__ i32x4 block_exclusive_scan4(i32x4 v, i32x4& total, i32x4* wave_tot) {
    constexpr int NW = THREADS / kWave;
    const int lane = threadIdx.x % kWave;
    const int w = threadIdx.x / kWave;
    i32x4 incl;
#pragma unroll
    for (int c = 0; c < 4; ++c) incl[c] = wave_inclusive_sum(v[c]);
    if (lane == kWave - 1) wave_tot[w] = incl;
    __syncthreads();
    i32x4 before = {0, 0, 0, 0};
    total = (i32x4){0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        if (i < w) before += wave_tot[i];
        total += wave_tot[i];
    }
    __syncthreads();  // wave_tot may be reused by the caller's next tile
    return before + incl - v;
}

// 2. Workgroup c scans expert column group c (4 experts, one int4) down the
// nb histogram rows: rows become exclusive prefixes, totals[4c..4c+3] the sums.
constexpr int kScanThreads = 256;
constexpr int kScanRowsPerLane = 8;

__global__ __launch_bounds__(kScanThreads) void route_scan_kernel(int32_t* __restrict__ block_counts, int nb,
                                                                  int Epad, int32_t* __restrict__ totals) {
    __shared__ i32x4 wave_tot[kScanThreads / kWave];
    const int Q = Epad / 4;
    i32x4* col = reinterpret_cast<i32x4*>(block_counts) + blockIdx.x;
    i32x4 carry = {0, 0, 0, 0};
    for (int base = 0; base < nb; base += kScanThreads * kScanRowsPerLane) {
        const int r0 = base + threadIdx.x * kScanRowsPerLane;
        i32x4 v[kScanRowsPerLane];
        i32x4 sum = {0, 0, 0, 0};
#pragma unroll
        for (int u = 0; u < kScanRowsPerLane; ++u) {
            v[u] = (r0 + u < nb) ? col[(size_t)(r0 + u) * Q] : (i32x4){0, 0, 0, 0};
            sum += v[u];
        }
        i32x4 tile_total;
        i32x4 run = carry + block_exclusive_scan4<kScanThreads>(sum, tile_total, wave_tot);
#pragma unroll
        for (int u = 0; u < kScanRowsPerLane; ++u) {
            if (r0 + u < nb) col[(size_t)(r0 + u) * Q] = run;
            run += v[u];
        }
        carry += tile_total;
    }
    if (threadIdx.x == 0) reinterpret_cast<i32x4*>(totals)[blockIdx.x] = carry;
}

// 3. Per workgroup of step 1: offsets from the totals (LDS scan), then
// dest = offset[e] + prefix[b][e] + rank for each of its slots.  With LIST
// each slot also gets its entry in the row list of its token group g:
// position gcum_g[e] + (tokens of group g before it that picked e), where
// gcum_g is the exclusive scan over experts of the group's own counts.
constexpr int kPlaceThreads = 256;
constexpr int kPlaceSlots = kChunk * kKMax / kPlaceThreads;  // slots per lane, at most

template <bool LIST>
__global__ __launch_bounds__(kPlaceThreads) void route_place_kernel(
    const int32_t* __restrict__ prefix, const int32_t* __restrict__ totals, int tok_per_block, int T, int E, int k,
    int pad, const int32_t* __restrict__ topk_ids, int32_t* __restrict__ dest_of_src,
    int32_t* __restrict__ src_of_dest, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ expert_counts,
    RowGroups groups, int2* __restrict__ row_list) {
    __shared__ int32_t s_tot[kEMax];
    __shared__ int32_t s_pre[kEMax];
    __shared__ int32_t s_off[kEMax + 1];
    __shared__ int32_t s_gpre[LIST ? kEMax : 1];
    __shared__ int32_t s_glen[LIST ? kEMax : 1];
    __shared__ int32_t s_gcum[LIST ? kEMax + 1 : 1];

    const int Epad = (E + 3) & ~3;
    const int b = blockIdx.x;
    const int tok0 = b * tok_per_block;
    const int nslot = min(tok_per_block, T - tok0) * k;
    const int gj = LIST ? group_of_unit(groups, b / kPlaceRows) : 0;  // the token group holding this row
    // every load first: the slots (expert, rank), the totals, this row's prefix
    int my_e[kPlaceSlots], my_r[kPlaceSlots];
#pragma unroll
    for (int u = 0; u < kPlaceSlots; ++u) {
        const int s = threadIdx.x + u * kPlaceThreads;
        if (s < nslot) {
            my_e[u] = topk_ids[(size_t)tok0 * k + s];
            my_r[u] = dest_of_src[(size_t)tok0 * k + s];
        }
    }
    for (int e = threadIdx.x; e < E; e += kPlaceThreads) {
        s_tot[e] = totals[e];
        s_pre[e] = prefix[(size_t)b * Epad + e];
        if constexpr (LIST) {
            const int r0 = group_row(groups, gj), r1 = group_row(groups, gj + 1);
            const int gpre = prefix[(size_t)r0 * Epad + e];
            const int gend = r1 < groups.nb ? prefix[(size_t)r1 * Epad + e] : totals[e];
            s_gpre[e] = gpre;
            s_glen[e] = gend - gpre;
        }
    }
    __syncthreads();
    wave_exclusive_scan(s_tot, s_off, E, pad, 0);
    if constexpr (LIST) wave_exclusive_scan(s_glen, s_gcum, E, 1, 1);
    __syncthreads();
    if (b == 0) {
        for (int e = threadIdx.x; e <= E; e += kPlaceThreads) expert_offsets[e] = s_off[e];
        if (expert_counts != nullptr)
            for (int e = threadIdx.x; e < E; e += kPlaceThreads) expert_counts[e] = s_tot[e];
    }
    mark_padding<kPlaceThreads>(s_tot, s_off, E, pad, b, gridDim.x, src_of_dest);
#pragma unroll
    for (int u = 0; u < kPlaceSlots; ++u) {
        const int s = threadIdx.x + u * kPlaceThreads;
        if (s < nslot) {
            const size_t gs = (size_t)tok0 * k + s;
            const int e = my_e[u];
            const int before = s_pre[e] + my_r[u];  // earlier tokens that picked e
            const int d = s_off[e] + before;
            dest_of_src[gs] = d;
            src_of_dest[d] = (int32_t)gs;
            if constexpr (LIST)
                row_list[(size_t)group_tok(groups, gj) * k + s_gcum[e] + (before - s_gpre[e])] =
                    make_int2(d, tok0 + s / k);
        }
    }
}

// 2+3 fused, for a small histogram matrix of count bytes: workgroup g owns
// kFusedRows consecutive top-k rows.  It sums every histogram row into column
// sums -- the totals and the prefix before its first row (and with LIST the
// prefixes at its token group's first and last row) -- keeps its own rows,
// scans the totals into offsets, and writes its slots.  Reading the whole
// matrix per workgroup costs L2 bandwidth instead of a third launch; the host
// picks this form only while the matrix is small (and T < 2^16, see below).
// With LIST each slot also gets its row-list entry (as in route_place_kernel).
//
// Lane layout: lane = rg * Qp + q, q = 16-byte column (16 experts), rg = row
// group; each lane sums rows rg, rg + RP, ...  A column's 16 count bytes are
// summed as 16-bit halves (bytes 0,2 and 1,3 of each word), which is exact
// while every total stays below 2^16, i.e. T < 2^16.  The row groups are
// reduced inside each wave by DPP row rotations and permlane swaps (lanes of
// one column sit Qp apart), then across the 16 waves through LDS.
constexpr int kFusedThreads = 1024;
constexpr int kFusedRows = kPlaceRows;
constexpr int kFusedSlots = kFusedRows * kChunk * kKMax / kFusedThreads;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kMaxRowVectors = kEMax / 16;

// With a COPY mode the same launch also expands the unit's token rows in
// token order (kCopyBf16: plain copy; kCopyFp8: quantised to E4M3 with one
// scale per `group` columns, as moe_expand_rows_fp8 does), over the slices of
// place_copy.h.  Every workgroup of a unit repeats the unit's scan+place
// (cheap: the histogram matrix is small on this path) and issues its row
// loads before it; the first (`owner`) also writes the unit's route outputs.
// The slot ranks then come from `ranks`, a workspace array, since the owner
// overwrites dest_of_src while its siblings may still read them.
static_assert(kPlaceCopyThreads == kFusedThreads, "the copying place step runs in the scan+place workgroup");

template <bool LIST, int QP, int COPY>
__device__ __forceinline__ void scan_place(
    const u32x4* __restrict__ rows8, int nb, int tok_per_row, int T, int E, int k, int pad,
    const int32_t* __restrict__ topk_ids, const int32_t* ranks, int32_t* dest_of_src,
    int32_t* __restrict__ src_of_dest, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ expert_counts,
    RowGroups groups, int2* __restrict__ row_list, const PlaceCopy& cp) {
    static_assert(!(LIST && COPY != kCopyNone), "the fused copy runs in token order, without the row list");
    const uint32_t chunks = COPY != kCopyNone ? cp.chunks : 1u;
    const uint32_t H16 = cp.H16;
    constexpr int NACC = LIST ? 4 : 2;
    __shared__ uint32_t part[NACC][kFusedWaves][kMaxRowVectors][8];
    __shared__ __attribute__((aligned(16))) uint8_t s_rows[kFusedRows][kEMax];
    __shared__ int32_t s_acc[NACC][kEMax];
    __shared__ int32_t s_off[kEMax + 1];
    __shared__ int32_t s_gcum[LIST ? kEMax + 1 : 1];
    __shared__ int32_t s_dest[COPY != kCopyNone ? kFusedRows * kChunk * kKMax : 1];

    constexpr int Qp = QP;                     // route_byte_row_vectors(E) <= 32
    // Only as many waves sum the histogram rows as give each lane about
    // kRowsPerLane rows (one batch of loads); the others skip the sums and
    // their lane reductions, which otherwise take most of the workgroup's
    // issue slots on small matrices.  sum_waves is wave-uniform.
    constexpr int kRowsPerLane = COPY != kCopyNone ? 1 : 4;
    const int sum_waves = min(kFusedWaves, max(1, (nb * Qp + kRowsPerLane * kWave - 1) / (kRowsPerLane * kWave)));
    const int RP = sum_waves * (kWave / Qp);  // row groups: lane (rg, q) sums rows rg, rg + RP, ...
    const bool summer = (int)(threadIdx.x / kWave) < sum_waves;
    const int q = threadIdx.x % Qp;
    const int rg = threadIdx.x / Qp;
    const int unit = (int)(blockIdx.x / chunks);
    const uint32_t chunk = blockIdx.x % chunks;
    const bool owner = chunk == 0;
    const int row0 = unit * kFusedRows;
    const int tok0 = row0 * tok_per_row;
    const int ntok = min(kFusedRows * tok_per_row, T - tok0);
    const int nslot = ntok * k;
    const int gj = LIST ? group_of_unit(groups, unit) : 0;  // the token group of this workgroup
    const int gfirst = LIST ? group_row(groups, gj) : 0;    // its rows [gfirst, gend)
    const int gend = LIST ? group_row(groups, gj + 1) : 0;

    // every independent load first: the row vectors to copy, the slots, then the histogram columns
    u32x4 xv[COPY != kCopyNone ? kCopyItems : 1];
    if constexpr (COPY != kCopyNone) {
#pragma unroll
        for (int m = 0; m < kCopyItems; ++m) {
            int tl;
            uint32_t col;
            xv[m] = (u32x4){0u, 0u, 0u, 0u};  // an absent item counts as zeros in a scale group
            if (copy_item<COPY>(cp, chunk, threadIdx.x + m * kFusedThreads, ntok, tl, col))
                xv[m] = load_stream(cp.x + (size_t)(tok0 + tl) * H16 + col);
        }
    }
    int my_e[kFusedSlots], my_r[kFusedSlots];
#pragma unroll
    for (int u = 0; u < kFusedSlots; ++u) {
        const int s = threadIdx.x + u * kFusedThreads;
        if (s < nslot) {
            my_e[u] = topk_ids[(size_t)tok0 * k + s];
            my_r[u] = ranks[(size_t)tok0 * k + s];
        }
    }
    // acc[a][2j] / acc[a][2j+1]: 16-bit sums of bytes (0,2) / (1,3) of word j,
    // over [0] every row, [1] the rows before row0, and with LIST [2] the
    // group's rows before row0, [3] the group's rows from row0 on (only the
    // waves that hold group rows do any work for these two)
    uint32_t acc[NACC][8];
#pragma unroll
    for (int a = 0; a < NACC; ++a)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[a][j] = 0;
    constexpr int kRowUnroll = COPY != kCopyNone ? 1 : 4;  // the copying form keeps registers for its rows
    if (summer) {
#pragma unroll kRowUnroll
        for (int row = rg; row < nb; row += RP) {
            const u32x4 w = rows8[(size_t)row * Qp + q];
            if (row >= row0 && row < row0 + kFusedRows) *reinterpret_cast<u32x4*>(&s_rows[row - row0][q * 16]) = w;
            uint32_t half[8];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                half[2 * j] = w[j] & 0x00FF00FFu;
                half[2 * j + 1] = (w[j] >> 8) & 0x00FF00FFu;
            }
            const uint32_t before_row0 = row < row0 ? 0xFFFFFFFFu : 0u;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                acc[0][j] += half[j];
                acc[1][j] += half[j] & before_row0;
            }
            if constexpr (LIST) {
                if (row >= gfirst && row < gend) {
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        acc[2][j] += half[j] & before_row0;
                        acc[3][j] += half[j] & ~before_row0;
                    }
                }
            }
        }
        // inside the wave: lanes of one column sit Qp apart
#pragma unroll
        for (int a = 0; a < NACC; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[a][j] = add_lanes<QP>(acc[a][j]);
        const int w = threadIdx.x / kWave;
        if ((int)(threadIdx.x % kWave) < Qp) {
#pragma unroll
            for (int a = 0; a < NACC; ++a)
#pragma unroll
                for (int j = 0; j < 8; ++j) part[a][w][q][j] = acc[a][j];
        }
    }
    __syncthreads();
    // lane (a, column, word): sum the summing waves, split the halves into experts
    for (int i = threadIdx.x; i < NACC * Qp * 8; i += kFusedThreads) {
        const int a = i / (Qp * 8);
        const int qq = (i / 8) % Qp;
        const int j = i % 8;
        uint32_t sum = 0;
#pragma unroll
        for (int v = 0; v < sum_waves; ++v) sum += part[a][v][qq][j];
        const int e = qq * 16 + (j / 2) * 4 + (j % 2);  // bytes 0/1 of word j/2; +2 for bytes 2/3
        if (e < E) s_acc[a][e] = (int32_t)(sum & 0xFFFFu);
        if (e + 2 < E) s_acc[a][e + 2] = (int32_t)(sum >> 16);
    }
    __syncthreads();
    wave_exclusive_scan(s_acc[0], s_off, E, pad, 0);
    if constexpr (LIST) wave_exclusive_scan(s_acc[2], s_gcum, E, 1, 1, s_acc[3]);  // the group's own counts
    __syncthreads();
    if (unit == 0 && owner) {
        for (int e = threadIdx.x; e <= E; e += kFusedThreads) expert_offsets[e] = s_off[e];
        if (expert_counts != nullptr)
            for (int e = threadIdx.x; e < E; e += kFusedThreads) expert_counts[e] = s_acc[0][e];
    }
    mark_padding<kFusedThreads>(s_acc[0], s_off, E, pad, blockIdx.x, gridDim.x, src_of_dest);
#pragma unroll
    for (int u = 0; u < kFusedSlots; ++u) {
        const int s = threadIdx.x + u * kFusedThreads;
        if (s < nslot) {
            const size_t gs = (size_t)tok0 * k + s;
            const int r = (s / k) / tok_per_row;
            const int e = my_e[u];
            int before = s_acc[1][e] + my_r[u];  // earlier tokens that picked e
            for (int r2 = 0; r2 < r; ++r2) before += s_rows[r2][e];
            const int d = s_off[e] + before;
            if (owner) {
                dest_of_src[gs] = d;
                src_of_dest[d] = (int32_t)gs;
            }
            if constexpr (COPY != kCopyNone) s_dest[s] = d;
            if constexpr (LIST)  // earlier tokens of the group that picked e: its rows before row0, then own
                row_list[(size_t)group_tok(groups, gj) * k + s_gcum[e] + s_acc[2][e] + (before - s_acc[1][e])] =
                    make_int2(d, tok0 + s / k);
        }
    }
    if constexpr (COPY == kCopyBf16) {
        __syncthreads();  // every destination of the unit is in s_dest
        u32x4* x_exp = static_cast<u32x4*>(cp.out);
#pragma unroll
        for (int m = 0; m < kCopyItems; ++m) {
            int tl;
            uint32_t col;
            if (copy_item<COPY>(cp, chunk, threadIdx.x + m * kFusedThreads, ntok, tl, col))
                for (int j = 0; j < k; ++j) store_stream(x_exp + (size_t)s_dest[tl * k + j] * H16 + col, xv[m]);
        }
    }
    if constexpr (COPY == kCopyFp8) {
        // a scale group is gl consecutive lanes of one token row (gl divides
        // H/8 and 64), present or absent as a whole
        __syncthreads();
        u32x2* q_out = static_cast<u32x2*>(cp.out);
#pragma unroll
        for (int m = 0; m < kCopyItems; ++m) {
            int tl;
            uint32_t col;
            const bool present = copy_item<COPY>(cp, chunk, threadIdx.x + m * kFusedThreads, ntok, tl, col);
            float f[8];
            unpack8(xv[m], f);
            const uint32_t amax_bits = group_abs_max(abs_max_bits8(f), cp.gl);
            if (present) {
                const BlockScale bs = block_scale(amax_bits, cp.mx);
                const u32x2 codes = quantize8_e4m3(f, bs.inv, bs.pre);
                const bool first_of_group = (threadIdx.x % (uint32_t)cp.gl) == 0;
                const uint32_t g = col / (uint32_t)cp.gl;
                for (int j = 0; j < k; ++j) {
                    const size_t d = (size_t)s_dest[tl * k + j];
                    __builtin_nontemporal_store(codes, q_out + d * H16 + col);
                    if (first_of_group) store_block_scale(cp.scales, d * cp.G + g, bs, cp.mx);
                }
            }
        }
    }
}

template <bool LIST, int QP>
__global__ __launch_bounds__(kFusedThreads) void route_scan_place_kernel(
    const u32x4* __restrict__ rows8, int nb, int tok_per_row, int T, int E, int k, int pad,
    const int32_t* __restrict__ topk_ids, int32_t* dest_of_src, int32_t* __restrict__ src_of_dest,
    int32_t* __restrict__ expert_offsets, int32_t* __restrict__ expert_counts, RowGroups groups,
    int2* __restrict__ row_list) {
    scan_place<LIST, QP, kCopyNone>(rows8, nb, tok_per_row, T, E, k, pad, topk_ids, dest_of_src, dest_of_src,
                                    src_of_dest, expert_offsets, expert_counts, groups, row_list, PlaceCopy{});
}

// The copying form: two workgroups per CU (at most 64 VGPRs), so that a grid
// of a few hundred workgroups runs in one round rather than two.
template <int QP, int COPY>
__global__ __launch_bounds__(kFusedThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void route_place_copy_kernel(
    const u32x4* __restrict__ rows8, int nb, int tok_per_row, int T, int E, int k, int pad,
    const int32_t* __restrict__ topk_ids, const int32_t* ranks, int32_t* dest_of_src,
    int32_t* __restrict__ src_of_dest, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ expert_counts,
    PlaceCopy cp) {
    scan_place<false, QP, COPY>(rows8, nb, tok_per_row, T, E, k, pad, topk_ids, ranks, dest_of_src, src_of_dest,
                                expert_offsets, expert_counts, RowGroups{}, nullptr, cp);
}

template <int QP>
void launch_scan_place(bool list, int nwg, const u32x4* rows8, int nb, int tok_per_row, const RouteArgs& a,
                       const int32_t* ranks, int2* row_list, hipStream_t stream) {
    PlaceCopy cp{};
    cp.chunks = 1;
    if (a.copy_out != nullptr) {
        // the caller checked H/8 <= kCopyItems * kFusedThreads for the quantising copy
        const int mode = a.copy_group > 0 ? kCopyFp8 : kCopyBf16;
        cp = make_place_copy(mode, kFusedRows * tok_per_row, a.copy_H, a.copy_group);
        cp.x = static_cast<const u32x4*>(a.copy_x);
        cp.out = a.copy_out;
        cp.scales = a.copy_scales;
        cp.mx = a.copy_mx;
        if (mode == kCopyFp8) {
            route_place_copy_kernel<QP, kCopyFp8><<<nwg * cp.chunks, kFusedThreads, 0, stream>>>(
                rows8, nb, tok_per_row, a.T, a.E, a.k, a.pad_to, a.topk_ids, ranks, a.dest_of_src, a.src_of_dest,
                a.expert_offsets, a.expert_counts, cp);
        } else {
            route_place_copy_kernel<QP, kCopyBf16><<<nwg * cp.chunks, kFusedThreads, 0, stream>>>(
                rows8, nb, tok_per_row, a.T, a.E, a.k, a.pad_to, a.topk_ids, ranks, a.dest_of_src, a.src_of_dest,
                a.expert_offsets, a.expert_counts, cp);
        }
    } else if (list) {
        route_scan_place_kernel<true, QP><<<nwg, kFusedThreads, 0, stream>>>(
            rows8, nb, tok_per_row, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.dest_of_src, a.src_of_dest,
            a.expert_offsets, a.expert_counts, a.groups, row_list);
    } else {
        route_scan_place_kernel<false, QP><<<nwg, kFusedThreads, 0, stream>>>(
            rows8, nb, tok_per_row, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.dest_of_src, a.src_of_dest,
            a.expert_offsets, a.expert_counts, a.groups, row_list);
    }
}

template <int G, int V>
hipError_t launch_route_gv(const RouteArgs& a, RouteVariant v, hipStream_t stream) {
    if (v == RouteVariant::SingleWorkgroup) {
        route_single_kernel<G, V><<<1, SingleShape<G>::THREADS, 0, stream>>>(
            a.logits, a.bias, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.topk_weights, a.expert_offsets, a.expert_counts,
            a.dest_of_src, a.src_of_dest);
        return hipGetLastError();
    }
    using S = TopkShape<G>;
    const int nb = (a.T + S::TOK - 1) / S::TOK;
    const int Epad = route_padded_experts(a.E);
    int32_t* counts = static_cast<int32_t*>(a.workspace);
    int32_t* totals = counts + (size_t)nb * Epad;
    // the slot ranks go to dest_of_src (finished in place), or with the fused
    // copy to the row-list area of the workspace
    const bool copy = v == RouteVariant::TwoPass && a.copy_out != nullptr;
    int32_t* ranks = copy ? reinterpret_cast<int32_t*>(static_cast<char*>(a.workspace) +
                                                        route_histogram_bytes(a.T, a.E))
                          : a.dest_of_src;
    if (v == RouteVariant::TwoPass)
        route_topk_kernel<G, V, true><<<nb, S::THREADS, 0, stream>>>(a.logits, a.bias, a.T, a.E, a.k, a.topk_ids,
                                                                     a.topk_weights, ranks, counts);
    else
        route_topk_kernel<G, V, false><<<nb, S::THREADS, 0, stream>>>(a.logits, a.bias, a.T, a.E, a.k, a.topk_ids,
                                                                      a.topk_weights, a.dest_of_src, counts);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    const bool list = a.row_list != nullptr;
    int2* row_list = reinterpret_cast<int2*>(a.row_list);
    if (v == RouteVariant::TwoPass) {
        const int nwg = (nb + kFusedRows - 1) / kFusedRows;
        const u32x4* rows8 = reinterpret_cast<const u32x4*>(counts);
        switch (route_byte_row_vectors(a.E)) {
            case 1: launch_scan_place<1>(list, nwg, rows8, nb, S::TOK, a, ranks, row_list, stream); break;
            case 2: launch_scan_place<2>(list, nwg, rows8, nb, S::TOK, a, ranks, row_list, stream); break;
            case 4: launch_scan_place<4>(list, nwg, rows8, nb, S::TOK, a, ranks, row_list, stream); break;
            case 8: launch_scan_place<8>(list, nwg, rows8, nb, S::TOK, a, ranks, row_list, stream); break;
            case 16: launch_scan_place<16>(list, nwg, rows8, nb, S::TOK, a, ranks, row_list, stream); break;
            default: launch_scan_place<32>(list, nwg, rows8, nb, S::TOK, a, ranks, row_list, stream); break;
        }
        return hipGetLastError();
    }
    route_scan_kernel<<<Epad / 4, kScanThreads, 0, stream>>>(counts, nb, Epad, totals);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    if (list)
        route_place_kernel<true><<<nb, kPlaceThreads, 0, stream>>>(
            counts, totals, S::TOK, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.dest_of_src, a.src_of_dest,
            a.expert_offsets, a.expert_counts, a.groups, row_list);
    else
        route_place_kernel<false><<<nb, kPlaceThreads, 0, stream>>>(
            counts, totals, S::TOK, a.T, a.E, a.k, a.pad_to, a.topk_ids, a.dest_of_src, a.src_of_dest,
            a.expert_offsets, a.expert_counts, a.groups, row_list);
    return hipGetLastError();
}

template <int G, int V>
hipError_t launch_topk_bytes_gv(const RouteArgs& a, int* nb_out, hipStream_t stream) {
    using S = TopkShape<G>;
    const int nb = (a.T + S::TOK - 1) / S::TOK;
    *nb_out = nb;
    route_topk_kernel<G, V, true, false><<<nb, S::THREADS, 0, stream>>>(
        a.logits, a.bias, a.T, a.E, a.k, a.topk_ids, a.topk_weights, nullptr, static_cast<int32_t*>(a.workspace));
    return hipGetLastError();
}

}  // namespace

int route_keys_per_lane(int E) { return E > 32 ? 8 : 4; }

int route_lanes_per_token(int E) {
    const int V = route_keys_per_lane(E);
    const int need = (E + V - 1) / V;
    int G = 1;
    while (G < need) G <<= 1;
    return G;
}

int route_quantising_place_max_h() { return 8 * kCopyItems * kFusedThreads; }

int route_tokens_per_block(int E) {
    const int G = route_lanes_per_token(E);
    return G >= 4 ? 16 : kWave / G;
}

RowGroups route_row_groups(int T, int E, int H) {
    RowGroups g;
    g.tb = route_tokens_per_block(E);
    g.nb = T > 0 ? (T + g.tb - 1) / g.tb : 0;
    g.units = std::max(1, (g.nb + kPlaceRows - 1) / kPlaceRows);
    g.T = T;
    // groups per XCD: enough that one group's source rows fit the L2 budget
    const int64_t per_xcd = ((int64_t)T * H * 2 + kXcds - 1) / kXcds;
    const int64_t sub = (per_xcd + kGroupSourceBytes - 1) / kGroupSourceBytes;
    g.n = kXcds * (int32_t)std::max<int64_t>(1, std::min<int64_t>(sub, kMaxGroupsPerXcd));
    return g;
}

RouteVariant route_pick_variant(int T, int E, RouteVariant requested) {
    if (T <= 0) return RouteVariant::SingleWorkgroup;  // writes the all-zero offsets
    switch (requested) {
        case RouteVariant::SingleWorkgroup:
            if (T <= kRouteFusedMaxTokens) return requested;
            break;
        case RouteVariant::TwoPass:  // its 16-bit column sums need T < 2^16
            return T <= kRouteTwoPassMaxTokens ? requested : RouteVariant::ThreePass;
        case RouteVariant::ThreePass:
            return requested;
        default:
            if (T <= kRouteSingleAutoMaxTokens) return RouteVariant::SingleWorkgroup;
            break;
    }
    const int tb = route_tokens_per_block(E);
    const size_t matrix = (size_t)((T + tb - 1) / tb) * route_byte_row_vectors(E) * 16;
    return matrix <= kRouteTwoPassMaxBytes && T <= kRouteTwoPassMaxTokens ? RouteVariant::TwoPass
                                                                          : RouteVariant::ThreePass;
}

hipError_t launch_route(const RouteArgs& a, RouteVariant variant, hipStream_t stream) {
    const RouteVariant v = route_pick_variant(a.T, a.E, variant);
    switch (route_lanes_per_token(a.E) * 16 + route_keys_per_lane(a.E)) {
        case 1 * 16 + 4: return launch_route_gv<1, 4>(a, v, stream);
        case 2 * 16 + 4: return launch_route_gv<2, 4>(a, v, stream);
        case 4 * 16 + 4: return launch_route_gv<4, 4>(a, v, stream);
        case 8 * 16 + 4: return launch_route_gv<8, 4>(a, v, stream);
        case 8 * 16 + 8: return launch_route_gv<8, 8>(a, v, stream);
        case 16 * 16 + 8: return launch_route_gv<16, 8>(a, v, stream);
        case 32 * 16 + 8: return launch_route_gv<32, 8>(a, v, stream);
        default: return launch_route_gv<64, 8>(a, v, stream);
    }
}

hipError_t launch_route_topk_bytes(const RouteArgs& a, int* nb, hipStream_t stream) {
    switch (route_lanes_per_token(a.E) * 16 + route_keys_per_lane(a.E)) {
        case 1 * 16 + 4: return launch_topk_bytes_gv<1, 4>(a, nb, stream);
        case 2 * 16 + 4: return launch_topk_bytes_gv<2, 4>(a, nb, stream);
        case 4 * 16 + 4: return launch_topk_bytes_gv<4, 4>(a, nb, stream);
        case 8 * 16 + 4: return launch_topk_bytes_gv<8, 4>(a, nb, stream);
        case 8 * 16 + 8: return launch_topk_bytes_gv<8, 8>(a, nb, stream);
        case 16 * 16 + 8: return launch_topk_bytes_gv<16, 8>(a, nb, stream);
        case 32 * 16 + 8: return launch_topk_bytes_gv<32, 8>(a, nb, stream);
        default: return launch_topk_bytes_gv<64, 8>(a, nb, stream);
    }
}

}  // namespace moe
