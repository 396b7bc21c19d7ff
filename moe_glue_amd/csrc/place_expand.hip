// The prefill route's second half and the expand in ONE launch: every
// workgroup places its own share of a token group's rows and copies them in
// destination order.
//
// "CuTeDSL at Perplexity", MoE dispatch/combine > Local: for many tokens the
// routing is split over many blocks, whose per-block counts are combined
// through global memory before the tokens are copied, on many more blocks,
// into the buffer the MoE GEMM reads.  Here the first launch (route.hip's
// top-k) leaves the top-k ids and, per 16-token block, one count byte per
// expert; this launch is the copy, and each of its workgroups derives the
// positions it needs itself instead of waiting for a separate place step
// (one launch and one round trip through memory fewer):
//
//   * the tokens are cut into 512 / S groups (RowGroups, at least 8), S
//     workgroups of 1024 lanes per group, so the whole grid is resident at
//     once at two workgroups per CU.  Group g is copied by XCD g % 8
//     (workgroup b runs on XCD b % 8): its source rows are read from HBM
//     about once and then served by that XCD's L2 (each is wanted k times).
//     A workgroup first issues cached loads of its 1/S of the group's source;
//   * it sums the count bytes over all blocks (the expert totals, hence the
//     offsets) and over the blocks before its group (the group's first row
//     inside each expert's segment);
//   * it reads the group's ids and builds, in LDS, a bitmap per expert of the
//     group's tokens that picked it; a slot's rank among the group's tokens of
//     its expert is the popcount of the bits below its token (the stable
//     order of the route: ascending token inside each expert), and its
//     position in the group's destination order is the group's count prefix
//     over the lower experts plus that rank.  Positions are cut into chunks
//     of one pass of a workgroup (Rc rows) and chunk q goes to workgroup
//     q % S, so the S workgroups of a group sweep its rows side by side;
//   * it copies its rows, then writes dest_of_src / src_of_dest for them.
//
// Every workgroup repeats its group's set-up (and all of them the histogram
// sums), so the set-up's length, not the copy, sets how much this saves:
// groups are kept small (a few hundred tokens), all set-up loads are issued
// before the first wait, and the map stores wait until after the copy.
#include "route_common.h"

#include <algorithm>

namespace moe {
namespace {

using namespace route_detail;

constexpr int kPeThreads = 1024;
constexpr int kPeWaves = kPeThreads / kWave;
constexpr int kPeSlots = kPeSlotsPerLane;        // group slots per lane
constexpr int kPeMaskWords = kPeMaskWordsMax;    // E * (group tokens / 64) bitmap words
constexpr int kPeRows = kPeRowsMax;              // rows one workgroup copies
constexpr int kPePrefetch = 4;                   // source vectors per lane touched up front
constexpr int kPeVectors = 1;                    // 16-byte vectors per lane per copy pass (1 beat 2 and 4)
constexpr int kPeDefaultS = 32;                  // workgroups per token group

template <int QP, int U>
__global__ __launch_bounds__(kPeThreads) __attribute__((amdgpu_waves_per_eu(8, 8))) void place_expand_kernel(
    const u32x4* __restrict__ rows8, int nb, int T, int E, int k, FastDiv div_k, int pad,
    const int32_t* __restrict__ topk_ids, RowGroups groups, int ls, int lrc, uint32_t H16, FastDiv div_h16,
    const u32x4* __restrict__ x, u32x4* __restrict__ x_exp, int32_t* __restrict__ dest_of_src,
    int32_t* __restrict__ src_of_dest, int32_t* __restrict__ expert_offsets, int32_t* __restrict__ expert_counts) {
    __shared__ uint32_t part[2][QP][8];  // column sums, two 16-bit halves per word
    __shared__ unsigned long long masks[kPeMaskWords];
    __shared__ uint16_t pc[kPeMaskWords];  // exclusive popcount prefix of each expert's bitmap words
    __shared__ int32_t s_tot[kEMax];
    __shared__ int32_t s_base[kEMax];
    __shared__ int32_t s_gcnt[kEMax];
    __shared__ int32_t s_off[kEMax + 1];
    __shared__ int32_t s_gcum[kEMax + 1];
    __shared__ int32_t s_tok[kPeRows];
    __shared__ int32_t s_dst[kPeRows];
    __shared__ int32_t s_slot[kPeRows];

    const int tid = threadIdx.x;
    const uint32_t S = 1u << ls, Rc = 1u << lrc;
    const uint32_t m = blockIdx.x / kXcds;
    const int g = (int)(m >> ls) * kXcds + (int)(blockIdx.x % kXcds);
    const uint32_t c = m & (S - 1);
    const int gt0 = group_tok(groups, g);
    const int gt1 = group_tok(groups, g + 1);
    const int gr0 = group_row(groups, g);
    const int ntok = gt1 - gt0;
    const int nslot = ntok * k;
    const int W = (ntok + kChunk - 1) / kChunk;  // bitmap words per expert

    // 1. Loads, in the order they are waited for (a wave's loads complete in
    // issue order): the first histogram rows of the summing lanes, the
    // group's ids, then this workgroup's 1/S of the group's source rows
    // (cached loads that only bring them into L2).
    // Lane (rg, q) sums rows rg, rg + RP, ... of 16-byte column q.
    constexpr int kRowsFirst = 4;
    const int sum_waves = min(kPeWaves, max(1, (nb * QP + kRowsFirst * kWave - 1) / (kRowsFirst * kWave)));
    const int RP = sum_waves * (kWave / QP);
    const int q = tid % QP;
    const int rg = tid / QP;
    const bool summer = tid / kWave < sum_waves;
    // Every load is unconditional (indices clamped into range, unwanted
    // values masked afterwards): loads behind divergent branches make the
    // compiler wait for each one before the next.
    u32x4 rowv[kRowsFirst];
#pragma unroll
    for (int u = 0; u < kRowsFirst; ++u) rowv[u] = rows8[(size_t)min(rg + u * RP, nb - 1) * QP + q];
    int my_e[kPeSlots];  // group-local slot s = tid + u * threads
    const int last_slot = T * k - 1;
#pragma unroll
    for (int u = 0; u < kPeSlots; ++u) my_e[u] = topk_ids[min(gt0 * k + tid + u * kPeThreads, last_slot)];
    for (int i = tid; i < E * W; i += kPeThreads) masks[i] = 0ull;
    for (int e = tid; e < E; e += kPeThreads) s_gcnt[e] = 0;
    for (int i = tid; i < 2 * QP * 8; i += kPeThreads) (&part[0][0][0])[i] = 0u;
    __syncthreads();  // bitmaps, counts and sums clear (the loads above are in flight; the
                      // source touches below would hold this barrier up while they queue)
    const uint32_t src_n = (uint32_t)ntok * H16;
    const uint32_t per = (src_n + S - 1) >> ls;
    const uint32_t pf0 = c * per;
    const uint32_t pf1 = min(src_n, pf0 + per);
    const uint32_t last_vec = (uint32_t)T * H16 - 1;
    const uint32_t* xw = reinterpret_cast<const uint32_t*>(x);
    uint32_t warm[kPePrefetch];
#pragma unroll
    for (int p = 0; p < kPePrefetch; ++p) {  // past this workgroup's slice: its last vector again
        const uint32_t j = min(pf0 + (uint32_t)(tid + p * kPeThreads), pf1 > 0 ? pf1 - 1 : 0u);
        warm[p] = xw[(size_t)min((uint32_t)gt0 * H16 + j, last_vec) * 4];  // one dword brings in the line
    }

    // 2. Column sums of the count bytes: [0] every row (the expert totals),
    // [1] the rows before the group (its first row in each expert's
    // segment), as 16-bit halves (bytes 0,2 and 1,3 of each word; exact
    // while T < 2^16).
    if (summer) {
        uint32_t acc[2][8];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[a][j] = 0;
        const auto add_row = [&](const u32x4& w, int row) {
            const uint32_t valid = row < nb ? 0xFFFFFFFFu : 0u;
            const uint32_t before = row < gr0 ? valid : 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const uint32_t lo = w[j] & 0x00FF00FFu, hi = (w[j] >> 8) & 0x00FF00FFu;
                acc[0][2 * j] += lo & valid;
                acc[0][2 * j + 1] += hi & valid;
                acc[1][2 * j] += lo & before;
                acc[1][2 * j + 1] += hi & before;
            }
        };
#pragma unroll
        for (int u = 0; u < kRowsFirst; ++u) add_row(rowv[u], rg + u * RP);
        for (int row = rg + kRowsFirst * RP; row < nb; row += RP) add_row(rows8[(size_t)row * QP + q], row);
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int j = 0; j < 8; ++j) acc[a][j] = add_lanes<QP>(acc[a][j]);
        if (tid % kWave < QP) {  // the wave's sums into the workgroup's (halves stay below 2^16)
#pragma unroll
            for (int a = 0; a < 2; ++a)
#pragma unroll
                for (int j = 0; j < 8; ++j) atomicAdd(&part[a][q][j], acc[a][j]);
        }
    }
    // 3. The group's per-expert token bitmaps and counts.
#pragma unroll
    for (int u = 0; u < kPeSlots; ++u) {
        const int s = tid + u * kPeThreads;
        if (s < nslot) {
            const int tl = (int)fastdiv((uint32_t)s, div_k);
            atomicOr(&masks[my_e[u] * W + (tl >> 6)], 1ull << (tl & 63));
            atomicAdd(&s_gcnt[my_e[u]], 1);
        }
    }
    __syncthreads();  // sums, bitmaps and group counts complete
    // 4. Side by side: wave 0 the expert totals and their (padded) offsets,
    // wave 1 the group's first rows and its destination order, the other
    // waves each bitmap word's popcount prefix inside its expert.  A wave
    // reads back what its own lanes wrote just before (LDS accesses of one
    // wave complete in order), so no barrier sits in between.
    const int wave = tid / kWave;
    if (wave < 2) {
        int32_t* dst = wave == 0 ? s_tot : s_base;
        for (int i = tid % kWave; i < QP * 8; i += kWave) {
            const int qq = i / 8;
            const int j = i % 8;
            const uint32_t sum = part[wave][qq][j];
            const int e = qq * 16 + (j / 2) * 4 + (j % 2);  // bytes 0/1 of word j/2; +2 for bytes 2/3
            if (e < E) dst[e] = (int32_t)(sum & 0xFFFFu);
            if (e + 2 < E) dst[e + 2] = (int32_t)(sum >> 16);
        }
        asm volatile("" ::: "memory");  // keep the scans' reads after these writes
        wave_exclusive_scan(s_tot, s_off, E, pad, 0);  // expert offsets (padded segments)
        wave_exclusive_scan(s_gcnt, s_gcum, E, 1, 1);  // the group's destination order
    } else {
        for (int i = tid - 2 * kWave; i < E * W; i += kPeThreads - 2 * kWave) {
            const int e = i / W;
            const int w = i - e * W;
            int run = 0;
            for (int w2 = 0; w2 < w; ++w2) run += __popcll(masks[e * W + w2]);
            pc[i] = (uint16_t)run;
        }
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += kPeThreads) expert_offsets[e] = s_off[e];
        if (expert_counts != nullptr)
            for (int e = tid; e < E; e += kPeThreads) expert_counts[e] = s_tot[e];
    }
    mark_padding<kPeThreads>(s_tot, s_off, E, pad, blockIdx.x, gridDim.x, src_of_dest);
    // 5. Every slot's position p in the group's destination order (the
    // group's count prefix over the lower experts plus the slot's rank among
    // the group's tokens of its expert); positions are cut into chunks of Rc
    // rows, chunk q goes to workgroup q % S as its row q / S * Rc + p % Rc.
#pragma unroll
    for (int u = 0; u < kPeSlots; ++u) {
        const int s = tid + u * kPeThreads;
        if (s < nslot) {
            const int e = my_e[u];
            const int tl = (int)fastdiv((uint32_t)s, div_k);
            const int w = tl >> 6;
            const unsigned long long below = (1ull << (tl & 63)) - 1ull;
            const int rank = (int)pc[e * W + w] + __popcll(masks[e * W + w] & below);
            const uint32_t p = (uint32_t)(s_gcum[e] + rank);
            const uint32_t qc = p >> lrc;
            if ((qc & (S - 1)) == c) {
                const uint32_t i = ((qc >> ls) << lrc) | (p & (Rc - 1));
                s_tok[i] = gt0 + tl;
                s_dst[i] = s_off[e] + s_base[e] + rank;
                s_slot[i] = gt0 * k + s;
            }
        }
    }
    __syncthreads();
    // 6. Copy this workgroup's rows, U vectors per lane per pass; the next
    // pass's vectors are loaded before this pass's are stored, so no load
    // waits behind an older store.
    const uint32_t nchunks = ((uint32_t)nslot + Rc - 1) >> lrc;
    const uint32_t mine = nchunks > c ? ((nchunks - c + S - 1) >> ls) : 0u;
    uint32_t rows = mine << lrc;
    const uint32_t last_end = (c + ((mine - 1) << ls) + 1) << lrc;  // end of this workgroup's last chunk
    if (mine > 0 && last_end > (uint32_t)nslot) rows -= last_end - (uint32_t)nslot;  // the group's last chunk
    const uint32_t items = rows * H16;
    const uint32_t step = kPeThreads * U;
    struct Batch {
        u32x4 v[U];
        uint32_t col[U];
        int32_t dst[U];
    };
    const auto fetch = [&](uint32_t i0, Batch& b) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = min(i0 + u * kPeThreads, items - 1);  // clamped: every read stays in bounds
            const uint32_t r = fastdiv(i, div_h16);
            b.col[u] = i - r * H16;
            b.dst[u] = s_dst[r];
            b.v[u] = x[(size_t)s_tok[r] * H16 + b.col[u]];  // cached: reused from L2
        }
    };
    const auto store = [&](uint32_t i0, const Batch& b) {
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (i0 + u * kPeThreads < items) store_stream(x_exp + (size_t)b.dst[u] * H16 + b.col[u], b.v[u]);
    };
    // two batches in turn: the next batch's loads are issued before this
    // batch's stores, so no load waits behind an older store and no batch
    // is copied between registers
    Batch ba, bb;
    uint32_t i0 = tid;
    if (i0 < items) fetch(i0, ba);
    while (i0 < items) {
        if (i0 + step < items) fetch(i0 + step, bb);
        store(i0, ba);
        i0 += step;
        if (i0 >= items) break;
        if (i0 + step < items) fetch(i0 + step, ba);
        store(i0, bb);
        i0 += step;
    }
    // 7. The maps of this workgroup's rows, after the copy: during the set-up
    // these stores would queue behind the source loads.
    for (uint32_t i = tid; i < rows; i += kPeThreads) {
        dest_of_src[s_slot[i]] = s_dst[i];
        src_of_dest[s_dst[i]] = s_slot[i];
    }
    // the touched source vectors are not needed themselves
#pragma unroll
    for (int p = 0; p < kPePrefetch; ++p) asm volatile("" ::"v"(warm[p]));
}

template <int QP>
hipError_t launch_qp(const PlaceExpandArgs& a, const PlaceExpandShape& sh, hipStream_t stream) {
    const uint32_t H16 = (uint32_t)a.H / 8;
    int ls = 0, lrc = 0;
    while ((1u << ls) < sh.S) ++ls;
    while ((1u << lrc) < sh.Rc) ++lrc;
    place_expand_kernel<QP, kPeVectors><<<sh.grid, kPeThreads, 0, stream>>>(
        static_cast<const u32x4*>(a.rows8), a.nb, a.T, a.E, a.k, make_fastdiv((uint32_t)a.k), a.pad_to, a.topk_ids,
        a.groups, ls, lrc, H16, make_fastdiv(H16), static_cast<const u32x4*>(a.x), static_cast<u32x4*>(a.x_expanded),
        a.dest_of_src, a.src_of_dest, a.expert_offsets, a.expert_counts);
    return hipGetLastError();
}

}  // namespace

static uint32_t pow2_floor(uint32_t v) {
    uint32_t p = 1;
    while (p * 2 <= v) p *= 2;
    return p;
}

PlaceExpandShape place_expand_shape(int T, int E, int k, int H, int workgroups_per_group) {
    PlaceExpandShape sh{};
    sh.ok = false;
    const int qp = route_byte_row_vectors(E);
    // 16-bit column sums need T < 2^16; a workgroup's items (rows * H/8) stay below 2^31
    if (T <= 0 || T > kRouteTwoPassMaxTokens || qp > 16 || (int64_t)kPeRowsMax * (H / 8) >= INT32_MAX) return sh;
    // S workgroups per group and 512 / S groups (at least 8, one per XCD): at
    // two 1024-lane workgroups per CU the whole grid is resident at once
    uint32_t S = pow2_floor(workgroups_per_group > 0 ? (uint32_t)workgroups_per_group : (uint32_t)kPeDefaultS);
    RowGroups g;
    g.tb = route_tokens_per_block(E);
    g.nb = (T + g.tb - 1) / g.tb;
    g.units = std::max(1, (g.nb + kPlaceRows - 1) / kPlaceRows);
    g.T = T;
    g.n = (int32_t)std::max<uint32_t>(kXcds, std::min<uint32_t>(kXcds * kMaxGroupsPerXcd, 512u / S));
    // more groups while one group's slots or bitmaps would not fit
    for (;;) {
        int max_tok = 0;
        for (int i = 0; i < g.n; ++i) max_tok = std::max(max_tok, group_tok(g, i + 1) - group_tok(g, i));
        const int words = E * ((max_tok + 63) / 64);
        if ((int64_t)max_tok * k <= (int64_t)kPeSlotsPerLane * 1024 && words <= kPeMaskWordsMax) break;
        if (g.n >= kXcds * kMaxGroupsPerXcd) return sh;
        g.n = std::min(kXcds * kMaxGroupsPerXcd, g.n * 2);
    }
    const uint32_t H16 = (uint32_t)H / 8;
    sh.Rc = pow2_floor(std::min<uint32_t>((uint32_t)kPeRowsMax,
                                          std::max<uint32_t>(1u, (uint32_t)(kPeThreads * kPeVectors) / H16)));
    // a workgroup copies at most kPeRowsMax rows
    int max_slots = 0;
    for (int i = 0; i < g.n; ++i) max_slots = std::max(max_slots, (group_tok(g, i + 1) - group_tok(g, i)) * k);
    for (;;) {
        const uint32_t nchunks = ((uint32_t)max_slots + sh.Rc - 1) / sh.Rc;
        if (((nchunks + S - 1) / S) * sh.Rc <= (uint32_t)kPeRowsMax) break;
        S *= 2;
    }
    sh.S = S;
    sh.groups = g;
    sh.grid = (uint32_t)((g.n + kXcds - 1) / kXcds) * kXcds * S;
    sh.ok = true;
    return sh;
}

hipError_t launch_place_expand(const PlaceExpandArgs& a, const PlaceExpandShape& sh, hipStream_t stream) {
    switch (route_byte_row_vectors(a.E)) {
        case 1: return launch_qp<1>(a, sh, stream);
        case 2: return launch_qp<2>(a, sh, stream);
        case 4: return launch_qp<4>(a, sh, stream);
        case 8: return launch_qp<8>(a, sh, stream);
        default: return launch_qp<16>(a, sh, stream);
    }
}

}  // namespace moe
