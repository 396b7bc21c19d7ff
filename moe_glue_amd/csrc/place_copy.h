// The slices of the copying place step (route.hip): when the route's
// scan+place launch also expands the rows in token order, the unit's tokens
// (kPlaceRows top-k rows) times H/8 columns are dealt to `chunks`
// workgroups of kPlaceCopyThreads lanes, kCopyItems 16-byte vectors per lane:
//   kCopyBf16  column slices of 2^cw_shift vectors across all the unit's
//              tokens (2^cw_shift * unit tokens = kCopyItems * lanes);
//   kCopyFp8   row slices of tpw whole token rows (tpw * H/8 <= kCopyItems *
//              lanes), so that a scale group is gl consecutive lanes of one
//              row and one workgroup writes all of an expanded row's scales.
// Item i of slice c is lane i % lanes, pass i / lanes.
#pragma once

#include <algorithm>
#include <stdint.h>

#include "device_common.h"

namespace moe {

constexpr int kCopyNone = 0;
constexpr int kCopyBf16 = 1;
constexpr int kCopyFp8 = 2;
constexpr int kCopyItems = 1;            // row vectors per lane (1 beat 2: finer slices)
constexpr int kPlaceCopyThreads = 1024;  // lanes per workgroup of the place step

struct PlaceCopy {
    const u32x4* x;
    void* out;        // u32x4 rows (bf16) or u32x2 rows (E4M3 codes)
    void* scales;     // kCopyFp8: [rows, G] fp32, or E8M0 bytes with mx
    bool mx;          // kCopyFp8: OCP microscaling scales (G = H/32, gl = 4)
    uint32_t H16;
    uint32_t G;       // kCopyFp8: scale groups per row
    int gl;           // kCopyFp8: lanes per scale group (group / 8)
    int cw_shift;     // kCopyBf16: 2^cw_shift vectors per column slice
    uint32_t tpw;     // kCopyFp8: token rows per slice
    FastDiv div_h16;  // kCopyFp8
    uint32_t chunks;  // slices per unit
};

// Slices for a unit of unit_tokens tokens (a power of two <= 2048) and rows of
// H bf16 (H % 8 == 0; for kCopyFp8 H/8 <= kCopyItems * kPlaceCopyThreads and
// group a power of two dividing H).
__host__ inline PlaceCopy make_place_copy(int mode, int unit_tokens, int H, int group) {
    PlaceCopy cp{};
    cp.H16 = (uint32_t)H / 8;
    constexpr uint32_t kItems = (uint32_t)(kCopyItems * kPlaceCopyThreads);
    if (mode == kCopyFp8) {
        cp.gl = group / 8;
        cp.G = (uint32_t)(H / group);
        cp.tpw = std::min<uint32_t>((uint32_t)unit_tokens, kItems / cp.H16);
        cp.div_h16 = make_fastdiv(cp.H16);
        cp.chunks = ((uint32_t)unit_tokens + cp.tpw - 1) / cp.tpw;
    } else {
        int s = 0;
        while (((uint32_t)unit_tokens << (s + 1)) <= kItems) ++s;
        cp.cw_shift = s;
        cp.chunks = (cp.H16 + (1u << s) - 1) >> s;
    }
    return cp;
}

// The unit-local token and the column of item `item` of slice `chunk`;
// false if the slice has no such item (a unit of ntok tokens).
template <int COPY>
__host__ __device__ __forceinline__ bool copy_item(const PlaceCopy& cp, uint32_t chunk, uint32_t item, int ntok,
                                                   int& tl, uint32_t& col) {
    if constexpr (COPY == kCopyFp8) {
        const uint32_t r = fastdiv(item, cp.div_h16);
        col = item - r * cp.H16;
        tl = (int)(chunk * cp.tpw + r);
        return r < cp.tpw && tl < ntok;
    } else {
        tl = (int)(item >> cp.cw_shift);
        col = (chunk << cp.cw_shift) + (item & ((1u << cp.cw_shift) - 1u));
        return tl < ntok && col < cp.H16;
    }
}

}  // namespace moe
