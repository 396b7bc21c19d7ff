// Host-side launchers of the gfx950 kernels.  Arguments arrive already
// validated by the C ABI layer (api.cpp); each launcher only picks a kernel
// variant and launch shape, enqueues it on `stream` and returns the launch
// status.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// ---------------------------------------------------------------- route
// Largest T the single-workgroup route accepts (four 64-token rank bitmaps),
// and the largest T it is chosen for automatically.
constexpr int kRouteFusedMaxTokens = 256;
constexpr int kRouteSingleAutoMaxTokens = 64;
// Largest histogram matrix (bytes) for which scan and place share one launch.
constexpr size_t kRouteTwoPassMaxBytes = 128 * 1024;

// Single workgroup; multi workgroup with the scan and place in one launch
// (TwoPass) or in two (ThreePass); Auto picks by T and the matrix size.
enum class RouteVariant { Auto = 0, SingleWorkgroup = 1, TwoPass = 2, ThreePass = 3 };

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
};

// Keys per lane (8 above 32 experts, else 4) and lanes that cooperate on one token.
int route_keys_per_lane(int E);
int route_lanes_per_token(int E);
// Tokens per workgroup of the multi-workgroup top-k (one workspace row each).
int route_tokens_per_block(int E);
// Experts padded to a multiple of 4 (one int4 per 4 experts in the workspace).
inline int route_padded_experts(int E) { return (E + 3) & ~3; }
// Workspace of the multi-workgroup route: one histogram row per top-k
// workgroup plus one row of totals.
inline size_t route_workspace_bytes(int T, int E) {
    const int tb = route_tokens_per_block(E);
    const size_t nb = (size_t)(T > 0 ? (T + tb - 1) / tb : 0);
    return (nb + 1) * (size_t)route_padded_experts(E) * sizeof(int32_t);
}
RouteVariant route_pick_variant(int T, int E, RouteVariant requested);

hipError_t launch_route(const RouteArgs& a, RouteVariant variant, hipStream_t stream);

// Route + expand in one launch for T <= kRouteSmallDispatchMaxTokens: every
// workgroup recomputes the routing in LDS and copies its share of the rows.
constexpr int kRouteSmallDispatchMaxTokens = 64;
hipError_t launch_route_expand_small(const RouteArgs& a, const void* x, int H, void* x_expanded, hipStream_t stream);

// ---------------------------------------------------- streaming row kernels
hipError_t launch_expand_rows(const void* x, const int32_t* dest_of_src, int T, int H, int k, void* x_expanded,
                              hipStream_t stream);
hipError_t launch_expand_rows_fp8(const void* x, const int32_t* dest_of_src, int T, int H, int k, int group,
                                  void* q_out, float* scales, hipStream_t stream);
hipError_t launch_swiglu(const void* h, int R, int I, void* act, hipStream_t stream);
hipError_t launch_combine(const void* y, const float* topk_weights, const int32_t* dest_of_src, int T, int H,
                          int k, void* out, hipStream_t stream);
hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t stream);

}  // namespace moe
