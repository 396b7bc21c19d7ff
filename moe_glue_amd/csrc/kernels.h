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
// Tokens per workgroup in the multi-workgroup route, and tokens per rank
// bitmap (one bit per token of a 64-bit word).
constexpr int kRouteTokensPerBlock = 64;
// Largest T the single-workgroup route accepts (four 64-token bitmaps).
constexpr int kRouteFusedMaxTokens = 256;

enum class RouteVariant { Auto = 0, SingleWorkgroup = 1, MultiWorkgroup = 2 };

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
};

// Experts padded to a multiple of 4 (one int4 per 4 experts in the workspace).
inline int route_padded_experts(int E) { return (E + 3) & ~3; }
inline int route_num_blocks(int T) { return (T + kRouteTokensPerBlock - 1) / kRouteTokensPerBlock; }
inline size_t route_workspace_bytes(int T, int E) {
    int nb = route_num_blocks(T);
    if (nb < 1) nb = 1;
    return (size_t)nb * (size_t)route_padded_experts(E) * sizeof(int32_t);
}
// Lanes that cooperate on one token: 4 keys per lane up to 256 experts, 8 beyond.
int route_lanes_per_token(int E);
RouteVariant route_pick_variant(int T, RouteVariant requested);

hipError_t launch_route(const RouteArgs& a, RouteVariant variant, hipStream_t stream);

// ---------------------------------------------------- streaming row kernels
hipError_t launch_expand_rows(const void* x, const int32_t* dest_of_src, int T, int H, int k, void* x_expanded,
                              hipStream_t stream);
hipError_t launch_swiglu(const void* h, int R, int I, void* act, hipStream_t stream);
hipError_t launch_combine(const void* y, const float* topk_weights, const int32_t* dest_of_src, int T, int H,
                          int k, void* out, hipStream_t stream);
hipError_t launch_copy_probe(const void* src, void* dst, size_t bytes, hipStream_t stream);

}  // namespace moe
