// Host check of the slices of the copying place step (place_copy.h): for
// both copy modes, unit sizes, row widths and partial units, every (token,
// column) of a unit is reached by exactly one (slice, item); for the FP8 mode
// every scale group is gl consecutive items, starting at a multiple of gl
// (so inside one wave), all present or all absent.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "place_copy.h"

using namespace moe;

static void fail(const char* what, long a, long b, long c) {
    std::printf("FAIL %s (%ld, %ld, %ld)\n", what, a, b, c);
    std::exit(1);
}

template <int MODE>
static void check(int unit_tokens, int ntok, int H, int group) {
    const PlaceCopy cp = make_place_copy(MODE, unit_tokens, H, group);
    const uint32_t H16 = (uint32_t)H / 8;
    const uint32_t items = (uint32_t)(kCopyItems * kPlaceCopyThreads);
    if (MODE == kCopyFp8 && (uint64_t)cp.tpw * H16 > items) fail("fp8 slice too large", unit_tokens, H, cp.tpw);
    if (MODE == kCopyBf16 && ((uint64_t)unit_tokens << cp.cw_shift) != items) fail("bf16 slice size", unit_tokens, H, cp.cw_shift);
    std::vector<int> seen((size_t)unit_tokens * H16, 0);
    for (uint32_t c = 0; c < cp.chunks; ++c) {
        for (uint32_t i = 0; i < items; ++i) {
            int tl;
            uint32_t col;
            const bool present = copy_item<MODE>(cp, c, i, ntok, tl, col);
            if (!present) continue;
            if (tl < 0 || tl >= ntok || col >= H16) fail("item out of range", unit_tokens, H, i);
            if (seen[(size_t)tl * H16 + col]++) fail("item reached twice", unit_tokens, H, i);
            if (MODE == kCopyFp8 && col % cp.gl == 0) {
                if (i % cp.gl != 0) fail("scale group not lane-aligned", H, group, i);
                for (uint32_t g = 1; g < (uint32_t)cp.gl; ++g) {
                    int tl2;
                    uint32_t col2;
                    if (!copy_item<MODE>(cp, c, i + g, ntok, tl2, col2) || tl2 != tl || col2 != col + g)
                        fail("scale group split", H, group, i);
                }
            }
        }
    }
    for (int t = 0; t < ntok; ++t)
        for (uint32_t col = 0; col < H16; ++col)
            if (seen[(size_t)t * H16 + col] != 1) fail("item never reached", unit_tokens, H, (long)t * H16 + col);
}

int main() {
    long cases = 0;
    for (int unit : {64, 128, 256})
        for (int H : {8, 16, 64, 136, 256, 520, 2048, 4096, 7168, 16384, 32768})
            for (int ntok : {unit, unit - 1, unit / 2 + 3, 1}) {
                check<kCopyBf16>(unit, ntok, H, 0);
                ++cases;
                if (H / 8 > kCopyItems * kPlaceCopyThreads) continue;  // the quantising fold needs whole rows
                for (int group = 8; group <= 512; group *= 2) {
                    if (H % group != 0) continue;
                    check<kCopyFp8>(unit, ntok, H, group);
                    ++cases;
                }
            }
    std::printf("ok %ld cases\n", cases);
    return 0;
}
