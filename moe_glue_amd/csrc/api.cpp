// The C ABI of moe_glue (declared in include/moe_glue.h): argument checks on
// the host, variant choice, launch.  Every check runs before the first HIP
// call, so a bad argument never reaches the device.
#include "moe_glue.h"

#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <atomic>

#include "kernels.h"
#include "moe_glue_testing.h"

namespace {

thread_local char g_last_error[512] = "";

moe_status fail(moe_status s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    std::vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return s;
}

moe_status ok() {
    g_last_error[0] = '\0';
    return MOE_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

moe_status from_hip(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Variant forcing for tests and measurements (moe_testing_force in
// include/moe_glue_testing.h): process-wide, read once per call.
std::atomic<int> g_force_route{0};  // 0 auto, 1 single, 2 two, 3 three
std::atomic<int> g_force_order{0};  // ExpandOrder + 1, 0 auto
std::atomic<int> g_force_wpg{0};    // workgroups per token group of the placing expand, 0 auto

moe::RouteVariant requested_route_variant() {
    switch (g_force_route.load(std::memory_order_relaxed)) {
        case 1: return moe::RouteVariant::SingleWorkgroup;
        case 2: return moe::RouteVariant::TwoPass;
        case 3: return moe::RouteVariant::ThreePass;
        default: return moe::RouteVariant::Auto;
    }
}

// Expand of moe_route_expand above the one-launch size:
//   Placed   the two-launch route's second launch is the expand itself
//            (place_expand.hip): each workgroup places and copies a share of
//            one token group's rows in destination order.  One launch and
//            one round trip through memory fewer than Grouped;
//   Grouped  destination order from a row list the route's place launch
//            writes (expand.hip): the form for batches outside Placed's
//            limits (three-launch route, E > 256, group sizes);
//   Fused    token order, copied by the route's scan+place launch itself
//            (two-launch route only), one launch less than Token;
//   Token    token order, a launch of its own after the route.
// Destination order pays from about 24576 expanded rows: token order
// scatters every token's k rows over k expert segments, a cost per expanded
// row; the destination-order forms' cost is mostly fixed.  Measured on this
// part with x coming from HBM (enough rotating input sets that no copy of x
// stays in the Infinity Cache), moe_route_expand per call with the row-list
// order against the copy in the place launch: at 16384 expanded rows the
// grouped call is 1.6-1.7 us behind (H = 2048 and 7168), from 24576 rows ahead
// at every width measured (H = 2048, 4096, 7168).
constexpr int64_t kGroupedExpandMinRows = 24576;

enum class ExpandOrder { Token = 0, Fused = 1, Grouped = 2, Placed = 3 };

constexpr int64_t kQuantisingFoldMaxBytes = 20ll << 20;  // E4M3 codes of moe_route_expand_fp8

int forced_order() { return g_force_order.load(std::memory_order_relaxed); }

// Placed runs every workgroup of the grid at once, each XCD on one or two
// token groups, so it pays while their source rows stay within the XCDs' L2
// and the histogram each workgroup sums stays small.  Measured per
// moe_route_expand call against the row-list order (T x H, E, k; x from
// HBM): 3072 x 2048 -1.4, 4096 x 2048 (the Qwen3-30B-A3B shape) -0.9,
// 4096 x 4096 (64, 6) -2.6, 6144 x 2048 -1.9, 4096 x 3072 +1.0, 8192 x 2048
// +1.9, 8192 x 7168 (256, 8) +38 us; and against the copy in the place launch
// (Fused): 768 x 4096 (64, 6) +0.3, 1023 x 4096 (64, 6) -1.6, 1024 x 2048
// -0.5, 2048 x 2048 -2.2, 1024 x 7168 (256, 8) -1.8, 2048 x 7168 (256, 8)
// -2.4 us.  Up to 24576 expanded rows 64 workgroups per group (one group per
// XCD) beat 32 by 0.1-0.6 us; at 32768 rows (Qwen3-30B-A3B) 32 beat 64 by 1.2.
// With one vector per lane in both copies the Fused crossover follows the
// expanded bytes: at H = 2048, k = 8, Placed minus Fused is +0.2 us at 832
// tokens (27 MB of expanded rows), -0.1 at 896 (29 MB), -0.35 at 960, -0.6
// at 1024, -0.4 at 1280; 1023 x 4096 (64, 6), 50 MB, -0.35.
constexpr int kPlacedMaxTokens = 6144;
constexpr int64_t kPlacedMaxSourceBytes = 32ll << 20;
constexpr int64_t kPlacedMinRows = 5120;
constexpr int64_t kPlacedMinExpandedBytes = 28ll << 20;
constexpr int64_t kPlacedWideGroupMaxRows = 24576;

ExpandOrder expand_order(int32_t T, int32_t E, int32_t k, int32_t H, moe::RouteVariant v,
                         moe::PlaceExpandShape* shape) {
    const bool two = v == moe::RouteVariant::TwoPass;
    if (v == moe::RouteVariant::SingleWorkgroup || T == 0) return ExpandOrder::Token;
    const int64_t rows = (int64_t)T * k;
    // without Placed: token order below the grouped expand's size, else grouped
    const ExpandOrder other = rows < kGroupedExpandMinRows ? (two ? ExpandOrder::Fused : ExpandOrder::Token)
                                                           : ExpandOrder::Grouped;
    switch (forced_order()) {
        case 1: return ExpandOrder::Token;
        case 2: return two ? ExpandOrder::Fused : ExpandOrder::Token;
        case 3: return ExpandOrder::Grouped;
        case 4: break;
        default:
            if (rows < kPlacedMinRows || rows * H * 2 < kPlacedMinExpandedBytes || T > kPlacedMaxTokens ||
                (int64_t)T * H * 2 > kPlacedMaxSourceBytes)
                return other;
    }
    if (two) {
        int wpg = g_force_wpg.load(std::memory_order_relaxed);
        if (wpg == 0) wpg = rows <= kPlacedWideGroupMaxRows ? 64 : 32;
        *shape = moe::place_expand_shape(T, E, k, H, wpg);
        if (shape->ok) return ExpandOrder::Placed;
    }
    return forced_order() == 4 ? ExpandOrder::Grouped : other;
}

moe_status check_route_sizes(int32_t T, int32_t E, int32_t k) {
    if (T < 0) return fail(MOE_ERR_SHAPE, "moe_route: T=%d is negative", T);
    if (E < 1) return fail(MOE_ERR_SHAPE, "moe_route: E=%d must be >= 1", E);
    if (k < 1 || k > E) return fail(MOE_ERR_SHAPE, "moe_route: k=%d must be in [1, E=%d]", k, E);
    if (E > MOE_E_MAX) return fail(MOE_ERR_UNSUPPORTED, "moe_route: E=%d exceeds %d", E, MOE_E_MAX);
    if (k > MOE_K_MAX) return fail(MOE_ERR_UNSUPPORTED, "moe_route: k=%d exceeds %d", k, MOE_K_MAX);
    if ((int64_t)T * E >= INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "moe_route: T*E=%lld too large",
                                                 (long long)T * E);
    return MOE_OK;
}

// bf16 row tensors: sizes, 16-byte rows (H % 8 == 0), element count in range.
moe_status check_rows(const char* fn, int32_t rows, int32_t width, const char* wname) {
    if (rows < 0) return fail(MOE_ERR_SHAPE, "%s: row count %d is negative", fn, rows);
    if (width < 1) return fail(MOE_ERR_SHAPE, "%s: %s=%d must be >= 1", fn, wname, width);
    if (width % 8 != 0)
        return fail(MOE_ERR_ALIGN, "%s: %s=%d: bf16 rows must be a multiple of 16 bytes (%s %% 8 == 0)", fn, wname,
                    width, wname);
    if ((int64_t)rows * (width / 8) >= INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "%s: %lld 16-byte vectors exceed the 2^31 limit", fn,
                    (long long)rows * (width / 8));
    return MOE_OK;
}

// Route argument checks shared by moe_route and moe_route_expand.
moe_status check_route_args(const char* fn, const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                            const int32_t* topk_ids, const float* topk_weights, const int32_t* expert_offsets,
                            const int32_t* dest_of_src, const int32_t* src_of_dest) {
    moe_status s = check_route_sizes(T, E, k);
    if (s != MOE_OK) return s;
    if (expert_offsets == nullptr) return fail(MOE_ERR_NULL, "%s: expert_offsets is NULL", fn);
    if (T > 0) {
        if (!logits || !topk_ids || !topk_weights || !dest_of_src || !src_of_dest)
            return fail(MOE_ERR_NULL, "%s: a required tensor pointer is NULL", fn);
        if (!aligned4(logits) || (bias && !aligned4(bias)))
            return fail(MOE_ERR_ALIGN, "%s: logits/bias must be 4-byte aligned", fn);
    }
    return MOE_OK;
}

// The histogram rows are needed by the multi-workgroup route; the row list
// only by moe_route_expand's grouped expand.
moe_status check_route_workspace(const char* fn, int32_t T, int32_t E, int32_t k, bool with_list,
                                 moe::RouteVariant v, const void* workspace, size_t workspace_bytes) {
    if (v == moe::RouteVariant::SingleWorkgroup) return MOE_OK;
    const size_t need = with_list ? moe::route_workspace_bytes(T, E, k) : moe::route_histogram_bytes(T, E);
    if (workspace == nullptr || workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given%s", fn, need, workspace_bytes,
                    workspace ? "" : " (NULL)");
    if (!aligned16(workspace)) return fail(MOE_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned", fn);
    return MOE_OK;
}

moe_status check_expand_args(const char* fn, const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H,
                             int32_t k, const uint16_t* x_expanded) {
    moe_status s = check_rows(fn, T, H, "H");
    if (s != MOE_OK) return s;
    if (k < 1 || k > MOE_K_MAX) return fail(MOE_ERR_SHAPE, "%s: k=%d must be in [1, %d]", fn, k, MOE_K_MAX);
    if ((int64_t)T * k >= INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k too large", fn);
    if (T == 0) return MOE_OK;
    if (!x || !dest_of_src || !x_expanded) return fail(MOE_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned16(x) || !aligned16(x_expanded))
        return fail(MOE_ERR_ALIGN, "%s: x and x_expanded must be 16-byte aligned", fn);
    return MOE_OK;
}

moe_status check_fp8_args(const char* fn, const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H,
                          int32_t k, int32_t group, const uint8_t* x_expanded, const float* scales) {
    moe_status s = check_rows(fn, T, H, "H");
    if (s != MOE_OK) return s;
    if (k < 1 || k > MOE_K_MAX) return fail(MOE_ERR_SHAPE, "%s: k=%d must be in [1, %d]", fn, k, MOE_K_MAX);
    if ((int64_t)T * k >= INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k too large", fn);
    if (group < 8 || group > 512 || (group & (group - 1)) != 0)
        return fail(MOE_ERR_UNSUPPORTED, "%s: group=%d must be a power of two in [8, 512]", fn, group);
    if (H % group != 0) return fail(MOE_ERR_SHAPE, "%s: H=%d is not a multiple of group=%d", fn, H, group);
    if (T == 0) return ok();
    if (!x || !dest_of_src || !x_expanded || !scales) return fail(MOE_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(x_expanded) & 7u) != 0 || !aligned4(scales))
        return fail(MOE_ERR_ALIGN, "%s: x must be 16-byte, codes 8-byte and scales 4-byte aligned", fn);
    return MOE_OK;
}

moe_status check_mxfp8_args(const char* fn, const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H,
                            int32_t k, const uint8_t* x_expanded, const uint8_t* scales) {
    moe_status s = check_rows(fn, T, H, "H");
    if (s != MOE_OK) return s;
    if (k < 1 || k > MOE_K_MAX) return fail(MOE_ERR_SHAPE, "%s: k=%d must be in [1, %d]", fn, k, MOE_K_MAX);
    if ((int64_t)T * k >= INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: T*k too large", fn);
    if (H % 32 != 0) return fail(MOE_ERR_SHAPE, "%s: H=%d is not a multiple of the 32-column block", fn, H);
    if (T == 0) return MOE_OK;
    if (!x || !dest_of_src || !x_expanded || !scales) return fail(MOE_ERR_NULL, "%s: NULL tensor pointer", fn);
    if (!aligned16(x) || (reinterpret_cast<uintptr_t>(x_expanded) & 7u) != 0)
        return fail(MOE_ERR_ALIGN, "%s: x must be 16-byte and codes 8-byte aligned", fn);
    return MOE_OK;
}

moe_status check_pad(const char* fn, int32_t T, int32_t E, int32_t k, int32_t pad_to) {
    if (pad_to < 1) return fail(MOE_ERR_SHAPE, "%s: pad_to=%d must be >= 1", fn, pad_to);
    if (pad_to > MOE_PAD_MAX) return fail(MOE_ERR_UNSUPPORTED, "%s: pad_to=%d exceeds %d", fn, pad_to, MOE_PAD_MAX);
    if ((int64_t)T * k + (int64_t)E * (pad_to - 1) >= INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "%s: padded rows exceed the 2^31 limit", fn);
    return MOE_OK;
}

moe_status route_impl(const char* fn, const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                      int32_t pad_to, int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                      int32_t* expert_counts, int32_t* dest_of_src, int32_t* src_of_dest, void* workspace,
                      size_t workspace_bytes, void* stream) {
    moe_status s = check_route_args(fn, logits, bias, T, E, k, topk_ids, topk_weights, expert_offsets, dest_of_src,
                                    src_of_dest);
    if (s != MOE_OK) return s;
    s = check_pad(fn, T, E, k, pad_to);
    if (s != MOE_OK) return s;
    const moe::RouteVariant v = moe::route_pick_variant(T, E, requested_route_variant());
    s = check_route_workspace(fn, T, E, k, false, v, workspace, workspace_bytes);
    if (s != MOE_OK) return s;
    moe::RouteArgs a{logits, bias, T, E, k, topk_ids, topk_weights, expert_offsets, expert_counts,
                     dest_of_src, src_of_dest, workspace, pad_to, nullptr, {}};
    return from_hip(moe::launch_route(a, v, static_cast<hipStream_t>(stream)), fn);
}

// moe_route_expand (pad_to = 1) and moe_route_expand_padded, for the
// caller's workspace or the built-in scratch.
moe_status route_expand_impl(const char* fn, const float* logits, const float* bias, int32_t T, int32_t E,
                             int32_t k, int32_t pad_to, const uint16_t* x, int32_t H, int32_t* topk_ids,
                             float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts,
                             int32_t* dest_of_src, int32_t* src_of_dest, uint16_t* x_expanded, void* workspace,
                             size_t workspace_bytes, void* stream) {
    moe_status s = check_route_args(fn, logits, bias, T, E, k, topk_ids, topk_weights,
                                    expert_offsets, dest_of_src, src_of_dest);
    if (s != MOE_OK) return s;
    s = check_pad(fn, T, E, k, pad_to);
    if (s != MOE_OK) return s;
    s = check_expand_args(fn, x, dest_of_src, T, H, k, x_expanded);
    if (s != MOE_OK) return s;
    const moe::RouteVariant requested = requested_route_variant();
    const hipStream_t st = static_cast<hipStream_t>(stream);
    moe::RouteArgs a{logits, bias, T, E, k, topk_ids, topk_weights, expert_offsets, expert_counts,
                     dest_of_src, src_of_dest, workspace, pad_to, /*row_list=*/nullptr, {}};
    if (T <= moe::kRouteSmallDispatchMaxTokens && requested == moe::RouteVariant::Auto) {
        a.copy_x = x;
        a.copy_out = x_expanded;
        a.copy_H = H;
        return from_hip(moe::launch_route_expand_small(a, st), fn);
    }
    const moe::RouteVariant v = moe::route_pick_variant(T, E, requested);
    s = check_route_workspace(fn, T, E, k, true, v, workspace, workspace_bytes);
    if (s != MOE_OK) return s;
    moe::PlaceExpandShape shape{};
    const ExpandOrder order = expand_order(T, E, k, H, v, &shape);
    if (order == ExpandOrder::Placed) {
        // top-k with count-byte rows, then placement and copy in one launch
        int nb = 0;
        s = from_hip(moe::launch_route_topk_bytes(a, &nb, st), fn);
        if (s != MOE_OK) return s;
        moe::PlaceExpandArgs pa{workspace, nb, T, E, k, H, pad_to, topk_ids, shape.groups, x, x_expanded,
                                dest_of_src, src_of_dest, expert_offsets, expert_counts};
        return from_hip(moe::launch_place_expand(pa, shape, st), fn);
    }
    // otherwise the multi-workgroup route either lists the rows per token
    // group for the destination-order expand, or copies them itself in token
    // order; the row list holds the real rows only, so padding rows stay
    // untouched exactly as moe_expand_rows leaves them
    if (order == ExpandOrder::Grouped) {
        a.row_list = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + moe::route_histogram_bytes(T, E));
        a.groups = moe::route_row_groups(T, E, H);
    } else if (order == ExpandOrder::Fused) {
        a.copy_x = x;
        a.copy_out = x_expanded;
        a.copy_H = H;
    }
    s = from_hip(moe::launch_route(a, v, st), fn);
    if (s != MOE_OK || T == 0 || order == ExpandOrder::Fused) return s;
    if (order == ExpandOrder::Grouped)
        return from_hip(moe::launch_expand_grouped(x, a.row_list, a.groups, H, k, x_expanded, st), fn);
    return from_hip(moe::launch_expand_rows(x, dest_of_src, T, H, k, x_expanded, st), fn);
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "MOE_OK";
        case MOE_ERR_NULL: return "MOE_ERR_NULL";
        case MOE_ERR_SHAPE: return "MOE_ERR_SHAPE";
        case MOE_ERR_ALIGN: return "MOE_ERR_ALIGN";
        case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
        case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
        case MOE_ERR_HIP: return "MOE_ERR_HIP";
    }
    return "MOE_ERR_UNKNOWN";
}

const char* moe_last_error(void) { return g_last_error; }

size_t moe_route_workspace_bytes(int32_t T, int32_t E, int32_t k) {
    if (check_route_sizes(T, E, k) != MOE_OK) return 0;
    return moe::route_workspace_bytes(T, E, k);
}


moe_status moe_route(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k, int32_t* topk_ids,
                     float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts, int32_t* dest_of_src,
                     int32_t* src_of_dest, void* workspace, size_t workspace_bytes, void* stream) {
    return route_impl("moe_route", logits, bias, T, E, k, 1, topk_ids, topk_weights, expert_offsets, expert_counts,
                      dest_of_src, src_of_dest, workspace, workspace_bytes, stream);
}

size_t moe_route_padded_rows(int32_t T, int32_t E, int32_t k, int32_t pad_to) {
    if (check_route_sizes(T, E, k) != MOE_OK || check_pad("moe_route_padded_rows", T, E, k, pad_to) != MOE_OK)
        return 0;
    return (size_t)T * k + (size_t)E * (pad_to - 1);
}

moe_status moe_route_padded(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k, int32_t pad_to,
                            int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts,
                            int32_t* dest_of_src, int32_t* src_of_dest, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return route_impl("moe_route_padded", logits, bias, T, E, k, pad_to, topk_ids, topk_weights, expert_offsets,
                      expert_counts, dest_of_src, src_of_dest, workspace, workspace_bytes, stream);
}

moe_status moe_expand_rows(const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H, int32_t k,
                           uint16_t* x_expanded, void* stream) {
    moe_status s = check_expand_args("moe_expand_rows", x, dest_of_src, T, H, k, x_expanded);
    if (s != MOE_OK) return s;
    if (T == 0) return ok();
    return from_hip(moe::launch_expand_rows(x, dest_of_src, T, H, k, x_expanded, static_cast<hipStream_t>(stream)),
                    "moe_expand_rows launch");
}

moe_status moe_route_expand(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                            const uint16_t* x, int32_t H, int32_t* topk_ids, float* topk_weights,
                            int32_t* expert_offsets, int32_t* expert_counts, int32_t* dest_of_src,
                            int32_t* src_of_dest, uint16_t* x_expanded, void* workspace, size_t workspace_bytes,
                            void* stream) {
    return route_expand_impl("moe_route_expand", logits, bias, T, E, k, 1, x, H, topk_ids, topk_weights,
                             expert_offsets, expert_counts, dest_of_src, src_of_dest, x_expanded, workspace,
                             workspace_bytes, stream);
}

size_t moe_noalloc_scratch_bytes(void) { return moe::kNoAllocScratchBytes; }

moe_status moe_route_expand_noalloc(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                                    const uint16_t* x, int32_t H, int32_t* topk_ids, float* topk_weights,
                                    int32_t* expert_offsets, int32_t* expert_counts, int32_t* dest_of_src,
                                    int32_t* src_of_dest, uint16_t* x_expanded, void* stream) {
    const char* fn = "moe_route_expand_noalloc";
    // every argument check and the size limit before the first HIP call
    moe_status s = check_route_args(fn, logits, bias, T, E, k, topk_ids, topk_weights, expert_offsets, dest_of_src,
                                    src_of_dest);
    if (s != MOE_OK) return s;
    s = check_expand_args(fn, x, dest_of_src, T, H, k, x_expanded);
    if (s != MOE_OK) return s;
    const size_t need = moe::route_workspace_bytes(T, E, k);
    if (need > moe::kNoAllocScratchBytes)
        return fail(MOE_ERR_UNSUPPORTED, "%s: T=%d E=%d k=%d needs %zu bytes of workspace; the built-in scratch "
                    "holds %zu (use moe_route_expand with a caller workspace)", fn, T, E, k, need,
                    moe::kNoAllocScratchBytes);
    void* ws = nullptr;
    s = from_hip(moe::noalloc_scratch(stream, &ws), "moe_route_expand_noalloc: scratch address");
    if (s != MOE_OK) return s;
    return route_expand_impl(fn, logits, bias, T, E, k, 1, x, H, topk_ids, topk_weights, expert_offsets,
                             expert_counts, dest_of_src, src_of_dest, x_expanded, ws, moe::kNoAllocScratchBytes,
                             stream);
}

moe_status moe_route_expand_padded(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                                   int32_t pad_to, const uint16_t* x, int32_t H, int32_t* topk_ids,
                                   float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts,
                                   int32_t* dest_of_src, int32_t* src_of_dest, uint16_t* x_expanded,
                                   void* workspace, size_t workspace_bytes, void* stream) {
    return route_expand_impl("moe_route_expand_padded", logits, bias, T, E, k, pad_to, x, H, topk_ids, topk_weights,
                             expert_offsets, expert_counts, dest_of_src, src_of_dest, x_expanded, workspace,
                             workspace_bytes, stream);
}

moe_status moe_expand_rows_fp8(const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H, int32_t k,
                               int32_t group, uint8_t* x_expanded, float* scales, void* stream) {
    const char* fn = "moe_expand_rows_fp8";
    moe_status s = check_fp8_args(fn, x, dest_of_src, T, H, k, group, x_expanded, scales);
    if (s != MOE_OK || T == 0) return s;
    return from_hip(moe::launch_expand_rows_fp8(x, dest_of_src, T, H, k, group, x_expanded, scales,
                                                static_cast<hipStream_t>(stream)),
                    "moe_expand_rows_fp8 launch");
}

moe_status moe_expand_rows_mxfp8(const uint16_t* x, const int32_t* dest_of_src, int32_t T, int32_t H, int32_t k,
                                 uint8_t* x_expanded, uint8_t* scales, void* stream) {
    moe_status s = check_mxfp8_args("moe_expand_rows_mxfp8", x, dest_of_src, T, H, k, x_expanded, scales);
    if (s != MOE_OK) return s;
    if (T == 0) return ok();
    return from_hip(moe::launch_expand_rows_mxfp8(x, dest_of_src, T, H, k, x_expanded, scales,
                                                  static_cast<hipStream_t>(stream)),
                    "moe_expand_rows_mxfp8 launch");
}

}  // extern "C"

namespace {

// moe_route_expand_fp8 / moe_route_expand_mxfp8: the route (padded for
// pad_to > 1), then the quantising expand with fp32 scales per `group`
// columns or, with mx, E8M0 scales per 32 columns.  Arguments already checked
// except the route workspace.
moe_status route_expand_quant(const char* fn, const float* logits, const float* bias, int32_t T, int32_t E,
                              int32_t k, int32_t pad_to, const uint16_t* x, int32_t H, int32_t group, bool mx,
                              int32_t* topk_ids, float* topk_weights, int32_t* expert_offsets,
                              int32_t* expert_counts, int32_t* dest_of_src, int32_t* src_of_dest,
                              uint8_t* x_expanded, void* scales, void* workspace, size_t workspace_bytes,
                              void* stream) {
    const moe::RouteVariant requested = requested_route_variant();
    const hipStream_t st = static_cast<hipStream_t>(stream);
    moe::RouteArgs a{logits, bias, T, E, k, topk_ids, topk_weights, expert_offsets, expert_counts,
                     dest_of_src, src_of_dest, workspace, pad_to, /*row_list=*/nullptr, {}};
    const auto set_copy = [&]() {
        a.copy_x = x;
        a.copy_out = x_expanded;
        a.copy_H = H;
        a.copy_group = group;
        a.copy_scales = scales;
        a.copy_mx = mx;
    };
    if (T <= moe::kRouteSmallDispatchMaxTokens && requested == moe::RouteVariant::Auto) {
        set_copy();
        return from_hip(moe::launch_route_expand_small(a, st), fn);
    }
    const moe::RouteVariant v = moe::route_pick_variant(T, E, requested);
    moe_status s = check_route_workspace(fn, T, E, k, true, v, workspace, workspace_bytes);
    if (s != MOE_OK) return s;
    // The quantising copy folds into the two-launch route's place step when
    // one of its workgroups holds a whole row and the codes are small: measured
    // at H = 2048, k = 8, group 128, folding saves 2-3 us up to 16 MB of codes
    // (T = 1000) but costs 3 us at 33 MB and 9 us at 67 MB (the copy then runs
    // well below the separate quantising expand's rate).
    // A forced token order keeps the separate expand, a forced fused order
    // folds whenever possible (tests and measurements).
    const bool forced_token = forced_order() == 1;
    const bool forced_fold = forced_order() == 2;
    const bool small = (int64_t)T * k * H <= kQuantisingFoldMaxBytes;
    const bool fold = v == moe::RouteVariant::TwoPass && T > 0 && H <= moe::route_quantising_place_max_h() &&
                      !forced_token && (small || forced_fold);
    if (fold) set_copy();
    s = from_hip(moe::launch_route(a, v, st), fn);
    if (s != MOE_OK || T == 0 || fold) return s;
    if (mx)
        return from_hip(moe::launch_expand_rows_mxfp8(x, dest_of_src, T, H, k, x_expanded,
                                                      static_cast<uint8_t*>(scales), st), fn);
    return from_hip(moe::launch_expand_rows_fp8(x, dest_of_src, T, H, k, group, x_expanded,
                                                static_cast<float*>(scales), st), fn);
}

}  // namespace

extern "C" {

moe_status moe_route_expand_fp8(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                                int32_t pad_to, const uint16_t* x, int32_t H, int32_t group, int32_t* topk_ids,
                                float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts,
                                int32_t* dest_of_src, int32_t* src_of_dest, uint8_t* x_expanded, float* scales,
                                void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_route_expand_fp8";
    moe_status s = check_route_args(fn, logits, bias, T, E, k, topk_ids, topk_weights, expert_offsets, dest_of_src,
                                    src_of_dest);
    if (s != MOE_OK) return s;
    s = check_pad(fn, T, E, k, pad_to);
    if (s != MOE_OK) return s;
    s = check_fp8_args(fn, x, dest_of_src, T, H, k, group, x_expanded, scales);
    if (s != MOE_OK) return s;
    return route_expand_quant(fn, logits, bias, T, E, k, pad_to, x, H, group, false, topk_ids, topk_weights,
                              expert_offsets, expert_counts, dest_of_src, src_of_dest, x_expanded, scales, workspace,
                              workspace_bytes, stream);
}

moe_status moe_route_expand_mxfp8(const float* logits, const float* bias, int32_t T, int32_t E, int32_t k,
                                  int32_t pad_to, const uint16_t* x, int32_t H, int32_t* topk_ids,
                                  float* topk_weights, int32_t* expert_offsets, int32_t* expert_counts,
                                  int32_t* dest_of_src, int32_t* src_of_dest, uint8_t* x_expanded, uint8_t* scales,
                                  void* workspace, size_t workspace_bytes, void* stream) {
    const char* fn = "moe_route_expand_mxfp8";
    moe_status s = check_route_args(fn, logits, bias, T, E, k, topk_ids, topk_weights, expert_offsets, dest_of_src,
                                    src_of_dest);
    if (s != MOE_OK) return s;
    s = check_pad(fn, T, E, k, pad_to);
    if (s != MOE_OK) return s;
    s = check_mxfp8_args(fn, x, dest_of_src, T, H, k, x_expanded, scales);
    if (s != MOE_OK) return s;
    return route_expand_quant(fn, logits, bias, T, E, k, pad_to, x, H, 32, true, topk_ids, topk_weights,
                              expert_offsets, expert_counts, dest_of_src, src_of_dest, x_expanded, scales, workspace,
                              workspace_bytes, stream);
}

moe_status moe_swiglu(const uint16_t* h, int32_t R, int32_t I, uint16_t* act, void* stream) {
    moe_status s = check_rows("moe_swiglu", R, I, "I");
    if (s != MOE_OK) return s;
    if ((int64_t)R * (2 * (int64_t)I / 8) >= INT32_MAX)
        return fail(MOE_ERR_UNSUPPORTED, "moe_swiglu: R*2I too large");
    if (R == 0) return ok();
    if (!h || !act) return fail(MOE_ERR_NULL, "moe_swiglu: NULL tensor pointer");
    if (!aligned16(h) || !aligned16(act)) return fail(MOE_ERR_ALIGN, "moe_swiglu: h and act must be 16-byte aligned");
    return from_hip(moe::launch_swiglu(h, R, I, act, static_cast<hipStream_t>(stream)), "moe_swiglu launch");
}

moe_status moe_combine(const uint16_t* y, const float* topk_weights, const int32_t* dest_of_src, int32_t T,
                       int32_t H, int32_t k, uint16_t* out, void* stream) {
    moe_status s = check_rows("moe_combine", T, H, "H");
    if (s != MOE_OK) return s;
    if (k < 1 || k > MOE_K_MAX) return fail(MOE_ERR_SHAPE, "moe_combine: k=%d must be in [1, %d]", k, MOE_K_MAX);
    if ((int64_t)T * k >= INT32_MAX) return fail(MOE_ERR_UNSUPPORTED, "moe_combine: T*k too large");
    if (T == 0) return ok();
    if (!y || !topk_weights || !dest_of_src || !out) return fail(MOE_ERR_NULL, "moe_combine: NULL tensor pointer");
    if (!aligned16(y) || !aligned16(out)) return fail(MOE_ERR_ALIGN, "moe_combine: y and out must be 16-byte aligned");
    if (!aligned4(topk_weights)) return fail(MOE_ERR_ALIGN, "moe_combine: topk_weights must be 4-byte aligned");
    return from_hip(moe::launch_combine(y, topk_weights, dest_of_src, T, H, k, out, static_cast<hipStream_t>(stream)),
                    "moe_combine launch");
}

int moe_testing_force(int route_variant, int expand_order, int workgroups_per_group) {
    if (route_variant < 0 || route_variant > 3 || expand_order < 0 || expand_order > 4 || workgroups_per_group < 0 ||
        workgroups_per_group > 4096)
        return -1;
    g_force_route.store(route_variant, std::memory_order_relaxed);
    g_force_order.store(expand_order, std::memory_order_relaxed);
    g_force_wpg.store(workgroups_per_group, std::memory_order_relaxed);
    return 0;
}

moe_status moe_copy_probe(const void* src, void* dst, size_t bytes, void* stream) {
    if (bytes == 0) return ok();
    if (!src || !dst) return fail(MOE_ERR_NULL, "moe_copy_probe: NULL pointer");
    if (bytes % 16 != 0 || !aligned16(src) || !aligned16(dst))
        return fail(MOE_ERR_ALIGN, "moe_copy_probe: size and pointers must be multiples of 16 bytes");
    return from_hip(moe::launch_copy_probe(src, dst, bytes, static_cast<hipStream_t>(stream)), "moe_copy_probe launch");
}

moe_status moe_mix_probe(const void* src, void* dst, uint32_t cycles, uint32_t reads, uint32_t writes,
                         int32_t vectors_per_lane, int32_t threads, void* stream) {
    if (vectors_per_lane != 1 && vectors_per_lane != 2 && vectors_per_lane != 4)
        return fail(MOE_ERR_SHAPE, "moe_mix_probe: vectors_per_lane=%d must be 1, 2 or 4", vectors_per_lane);
    if (threads != 64 && threads != 256 && threads != 1024)
        return fail(MOE_ERR_SHAPE, "moe_mix_probe: threads=%d must be 64, 256 or 1024", threads);
    if (reads > 64 || writes > 64 || (uint64_t)cycles * (reads + writes) > (1u << 24))
        return fail(MOE_ERR_SHAPE, "moe_mix_probe: at most 64 reads and 64 writes per cycle and 2^24 waves");
    if (cycles == 0 || (reads == 0 && writes == 0)) return ok();
    if ((reads > 0 && !src) || !dst) return fail(MOE_ERR_NULL, "moe_mix_probe: NULL pointer");
    if (!aligned16(src) || !aligned16(dst)) return fail(MOE_ERR_ALIGN, "moe_mix_probe: pointers must be 16-byte aligned");
    return from_hip(moe::launch_mix_probe(src, dst, cycles, reads, writes, vectors_per_lane, threads,
                                          static_cast<hipStream_t>(stream)),
                    "moe_mix_probe launch");
}

}  // extern "C"
