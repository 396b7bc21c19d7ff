// Host-side launchers of the gfx950 kernels.  Arguments arrive already
// validated by the C ABI layer (api.cpp); each launcher only picks a kernel
// variant and launch shape, enqueues it on `stream` and returns the launch
// status.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe_glue.h"

namespace moe {

// ---------------------------------------------------------------- route
// Largest T the single-workgroup route accepts (four 64-token rank bitmaps),
// and the largest T it is chosen for automatically.
constexpr int kRouteFusedMaxTokens = 256;
constexpr int kRouteSingleAutoMaxTokens = 64;
// Largest histogram matrix (bytes, one count byte per expert and top-k row)
// for which scan and place share one launch, and the largest T (the column
// sums are formed in 16-bit halves).
constexpr size_t kRouteTwoPassMaxBytes = 128 * 1024;
constexpr int kRouteTwoPassMaxTokens = 65535;

// Single workgroup; multi workgroup with the scan and place in one launch
// (TwoPass) or in two (ThreePass); Auto picks by T and the matrix size.
enum class RouteVariant { Auto = 0, SingleWorkgroup = 1, TwoPass = 2, ThreePass = 3 };

// Token groups of the grouped expand.  Workgroups are dealt to the 8 XCDs
// round-robin, so workgroup b runs on XCD b % 8; XCD x copies the rows of
// groups x, x + 8, x + 16, ... one group after the other, and a group's
// source rows (about kGroupSourceBytes at most) stay in that XCD's L2.
// Group boundaries fall on whole scan+place workgroups ("units" of
// kPlaceRows top-k rows): group i starts at top-k row
// row(i) = min(nb, kPlaceRows * floor(i * units / n)).
constexpr int kXcds = 8;
constexpr int kPlaceRows = 4;
constexpr int64_t kGroupSourceBytes = 2 << 20;
constexpr int kMaxGroupsPerXcd = 16;
struct RowGroups {
    int32_t n;      // number of groups: kXcds * groups per XCD
    int32_t units;  // scan+place units
    int32_t nb;     // top-k rows
    int32_t tb;     // tokens per top-k row
    int32_t T;
};
// (32-bit unsigned arithmetic: units < 2^25 and n <= 128 keep every product
// below 2^32.)
__host__ __device__ inline int32_t group_row(const RowGroups& g, int i) {
    const uint32_t r = (uint32_t)kPlaceRows * ((uint32_t)i * (uint32_t)g.units / (uint32_t)g.n);
    return r < (uint32_t)g.nb ? (int32_t)r : g.nb;
}
__host__ __device__ inline int32_t group_tok(const RowGroups& g, int i) {
    const int64_t t = (int64_t)group_row(g, i) * g.tb;
    return t < g.T ? (int32_t)t : g.T;
}
// The group holding unit u: the last i with floor(i * units / n) <= u.
__host__ __device__ inline int32_t group_of_unit(const RowGroups& g, int u) {
    const uint32_t units = (uint32_t)g.units;
    const int32_t i = (int32_t)((((uint32_t)u + 1) * (uint32_t)g.n + units - 1) / units) - 1;
    return i < g.n - 1 ? i : g.n - 1;
}

struct RouteArgs {
    const float* logits;
    const float* bias;
    int T, E, k;
    int32_t* topk_ids;
    float* topk_weights;
    int32_t* expert_offsets;
    int32_t* expert_counts;
    int32_t* dest_of_src;
    int32_t* src_of_dest;
    void* workspace;
    int pad_to;  // expert segments padded to a multiple of pad_to rows (1: unpadded)
    // When set (multi-workgroup variants only): the expanded rows listed per
    // token group of `groups` for the grouped expand; entry = (dest row,
    // token), group i at [tok(i)*k, tok(i+1)*k), each group in dest-row order.
    int32_t* row_list;
    RowGroups groups;
    // When set (two-launch variant only, not with row_list): the place step
    // also copies x [T, copy_H] bf16 to copy_out in token order (the expand;
    // with copy_group > 0 quantised to E4M3 codes plus copy_scales, one scale
    // per copy_group columns: fp32 amax/448, or with copy_mx an E8M0 byte per
    // 32 columns), keeping the slot ranks in the workspace's
    // row-list area meanwhile.
    const void* copy_x;
    void* copy_out;
    int copy_H;
    int copy_group;
    void* copy_scales;  // float [rows, H/copy_group], or uint8_t E8M0 [rows, H/32] with copy_mx
    bool copy_mx;
};

// Keys per lane (8 above 32 experts, else 4) and lanes that cooperate on one token.
int route_keys_per_lane(int E);
int route_lanes_per_token(int E);
// Tokens per workgroup of the multi-workgroup top-k (one workspace row each).
int route_tokens_per_block(int E);
// Widest row (H) whose FP8 quantising copy the place step can take on: one
// workgroup holds at least one whole row.
int route_quantising_place_max_h();
// Experts padded to a multiple of 4 (one int4 per 4 experts in the workspace).
inline int route_padded_experts(int E) { return (E + 3) & ~3; }
// 16-byte vectors per byte histogram row (one count byte per expert): E/16
// rounded up to a power of two.
__host__ __device__ inline int route_byte_row_vectors(int E) {
    int p = 1;
    while (p * 16 < E) p <<= 1;
    return p;
}
// Workspace of the multi-workgroup route: one histogram row per top-k
// workgroup plus one row of totals, then (16-byte aligned) the row list of
// the grouped expand, T*k entries of two int32.
inline size_t route_histogram_bytes(int T, int E) {
    const int tb = route_tokens_per_block(E);
    const size_t nb = (size_t)(T > 0 ? (T + tb - 1) / tb : 0);
    return ((nb + 1) * (size_t)route_padded_experts(E) * sizeof(int32_t) + 15) & ~(size_t)15;
}
inline size_t route_workspace_bytes(int T, int E, int k) {
    return route_histogram_bytes(T, E) + (size_t)T * k * 2 * sizeof(int32_t);
}
// Groups for a batch of T tokens whose rows are H bf16 wide.
RowGroups route_row_groups(int T, int E, int H);
RouteVariant route_pick_variant(int T, int E, RouteVariant requested);

hipError_t launch_route(const RouteArgs& a, RouteVariant variant, hipStream_t stream);

// Route + expand in one launch for T <= kRouteSmallDispatchMaxTokens: every
// workgroup recomputes the routing in LDS and copies its share of the rows.
constexpr int kRouteSmallDispatchMaxTokens = 64;
// The copy is RouteArgs::copy_* (bf16, or E4M3 with copy_group > 0, MX scales with copy_mx); segments
// padded to pad_to rows.
hipError_t launch_route_expand_small(const RouteArgs& a, hipStream_t stream);

// The prefill route + expand in two launches (place_expand.hip): the top-k
// launch writes ids, weights and count-byte rows (no ranks); the second
// launch places and copies each token group's rows in destination order.
constexpr int kPeSlotsPerLane = 4;     // group slots <= 4 * 1024
constexpr int kPeMaskWordsMax = 2048;  // E * ceil(group tokens / 64) bitmap words
constexpr int kPeRowsMax = 512;        // rows one workgroup copies
struct PlaceExpandShape {
    bool ok;          // false: the shape is outside this path (use the row-list path)
    RowGroups groups;
    uint32_t S;       // workgroups per group
    uint32_t Rc;      // rows per chunk (one pass of a workgroup)
    uint32_t grid;
};
struct PlaceExpandArgs {
    const void* rows8;  // count-byte rows of the top-k launch (workspace)
    int nb;             // top-k rows
    int T, E, k, H, pad_to;
    const int32_t* topk_ids;
    RowGroups groups;
    const void* x;
    void* x_expanded;
    int32_t* dest_of_src;
    int32_t* src_of_dest;
    int32_t* expert_offsets;
    int32_t* expert_counts;
};
// Position of the (r+1)-th set bit of m (r < popcount(m)), by halving.
__host__ __device__ inline int select_bit(unsigned long long m, int r) {
    int pos = 0;
#pragma unroll
    for (int width = 32; width >= 1; width /= 2) {
        const unsigned long long low = m & ((1ull << width) - 1ull);
        const int c = __builtin_popcountll(low);
        if (r >= c) {
            r -= c;
            m >>= width;
            pos += width;
        } else {
            m = low;
        }
    }
    return pos;
}
// The shape for (T, E, k, H); workgroups_per_group = 0 picks the default.
PlaceExpandShape place_expand_shape(int T, int E, int k, int H, int workgroups_per_group);
hipError_t launch_place_expand(const PlaceExpandArgs& a, const PlaceExpandShape& sh, hipStream_t stream);
// The top-k launch of that path: ids, weights and count-byte rows (workspace
// front part) of every 16-token block; returns the number of rows in *nb.
hipError_t launch_route_topk_bytes(const RouteArgs& a, int* nb, hipStream_t stream);

// ---------------------------------------------------- streaming row kernels
hipError_t launch_expand_rows(const void* x, const int32_t* dest_of_src, int T, int H, int k, void* x_expanded,
                              hipStream_t stream);
// Expand in destination-row order from the route's row list (RouteArgs::row_list).
hipError_t launch_expand_grouped(const void* x, const int32_t* row_list, const RowGroups& groups, int H, int k,
                                 void* x_expanded, hipStream_t stream);
hipError_t launch_expand_rows_fp8(const void* x, const int32_t* dest_of_src, int T, int H, int k, int group,
                                  void* q_out, float* scales, hipStream_t stream);
// MXFP8: E4M3 codes with one E8M0 scale byte per block of 32 columns (H % 32 == 0).
hipError_t launch_expand_rows_mxfp8(const void* x, const int32_t* dest_of_src, int T, int H, int k, void* q_out,
                                    uint8_t* scales, hipStream_t stream);
hipError_t launch_swiglu(const void* h, int R, int I, void* act, hipStream_t stream);
hipError_t launch_combine(const void* y, const float* topk_weights, const int32_t* dest_of_src, int T, int H,
                          int k, void* out, hipStream_t stream);
hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t stream);
hipError_t launch_mix_probe(const void* src, void* dst, uint32_t cycles, uint32_t reads, uint32_t writes,
                            int vectors_per_lane, int threads, hipStream_t stream);

// ------------------------------------------------------- built-in scratch
// Bytes of the file-scope device array behind moe_route_expand_noalloc.
constexpr size_t kNoAllocScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
// Device address of that array on the device `stream` runs on (the current
// device for the null stream), looked up on the first call per device.
hipError_t noalloc_scratch(void* stream, void** out);

}  // namespace moe
