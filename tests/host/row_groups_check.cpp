// Host check of the token-group arithmetic behind moe_route_expand's grouped
// expand (kernels.h, route.hip, expand.hip):
//  * route_row_groups: n is a multiple of 8 (<= 128), group boundaries fall
//    on whole scan+place units, group_row(0) = 0, group_row(n) = nb, and
//    group_tok follows group_row;
//  * group_of_unit(u) is the group whose rows hold unit u;
//  * a model of the row-list positions the place steps compute (the group's
//    expert starts plus the group's earlier tokens of the same expert) fills
//    every group's slice exactly once, in destination-row order;
//  * the expand grid (groups dealt to XCDs, chunks of rows) covers every
//    (group, chunk) once;
//  * the workspace holds the byte histogram and the int32 histogram forms.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>

#include "kernels.h"

using namespace moe;

static void fail(const char* what, long a, long b, long c) {
    std::printf("FAIL %s (%ld, %ld, %ld)\n", what, a, b, c);
    std::exit(1);
}

static void check_groups(int T, int E, int H) {
    const RowGroups g = route_row_groups(T, E, H);
    const int tb = route_tokens_per_block(E);
    const int nb = (T + tb - 1) / tb;
    const int units = (nb + kPlaceRows - 1) / kPlaceRows;
    if (g.n % kXcds != 0 || g.n > kXcds * kMaxGroupsPerXcd) fail("group count", T, E, g.n);
    if (group_row(g, 0) != 0 || group_row(g, g.n) != nb) fail("group ends", T, E, g.n);
    for (int i = 0; i < g.n; ++i) {
        const int r0 = group_row(g, i), r1 = group_row(g, i + 1);
        if (r1 < r0 || (r0 % kPlaceRows != 0 && r0 != nb)) fail("group rows", T, i, r0);
        if (group_tok(g, i) != std::min(T, r0 * tb)) fail("group tokens", T, i, group_tok(g, i));
    }
    for (int u = 0; u < units; ++u) {
        const int i = group_of_unit(g, u);
        if (!(group_row(g, i) <= u * kPlaceRows && u * kPlaceRows < group_row(g, i + 1))) fail("unit group", T, u, i);
    }
}

// Random routing of T tokens, then the list positions of every slot as the
// scan+place step computes them; checks the slices and their order.
static void check_list(int T, int E, int k, int H, unsigned seed) {
    std::mt19937 rng(seed);
    const RowGroups g = route_row_groups(T, E, H);
    const int tb = g.tb;
    const int nb = (T + tb - 1) / tb;
    std::vector<int> ids((size_t)T * k), perm(E);
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) perm[e] = e;
        std::shuffle(perm.begin(), perm.end(), rng);
        for (int j = 0; j < k; ++j) ids[(size_t)t * k + j] = perm[j];
    }
    // per top-k row counts and ranks, column prefixes, offsets
    std::vector<int> cnt((size_t)nb * E, 0), rank((size_t)T * k);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int e = ids[(size_t)t * k + j];
            rank[(size_t)t * k + j] = cnt[(size_t)(t / tb) * E + e]++;
        }
    std::vector<long> pre((size_t)(nb + 1) * E, 0);
    for (int r = 0; r < nb; ++r)
        for (int e = 0; e < E; ++e) pre[(size_t)(r + 1) * E + e] = pre[(size_t)r * E + e] + cnt[(size_t)r * E + e];
    std::vector<long> off(E + 1, 0);
    for (int e = 0; e < E; ++e) off[e + 1] = off[e] + pre[(size_t)nb * E + e];
    const long R = (long)T * k;
    std::vector<long> list_dest(R, -1), list_tok(R, -1);
    for (int t = 0; t < T; ++t) {
        const int row = t / tb;
        const int gi = group_of_unit(g, row / kPlaceRows);
        const int g0 = group_row(g, gi), g1 = group_row(g, gi + 1);
        // the group's own counts and their exclusive scan over experts
        std::vector<long> gcum(E + 1, 0);
        for (int e = 0; e < E; ++e) gcum[e + 1] = gcum[e] + pre[(size_t)g1 * E + e] - pre[(size_t)g0 * E + e];
        for (int j = 0; j < k; ++j) {
            const int e = ids[(size_t)t * k + j];
            const long before = pre[(size_t)row * E + e] + rank[(size_t)t * k + j];
            const long d = off[e] + before;
            const long p = (long)group_tok(g, gi) * k + gcum[e] + (before - pre[(size_t)g0 * E + e]);
            if (p < (long)group_tok(g, gi) * k || p >= (long)group_tok(g, gi + 1) * k) fail("list slice", T, t, p);
            if (list_dest[p] != -1) fail("list position used twice", T, t, p);
            list_dest[p] = d;
            list_tok[p] = t;
        }
    }
    for (int i = 0; i < g.n; ++i)
        for (long p = (long)group_tok(g, i) * k + 1; p < (long)group_tok(g, i + 1) * k; ++p)
            if (list_dest[p] <= list_dest[p - 1]) fail("destination order", T, i, p);
    // the expand grid reaches every (group, chunk) once
    const uint32_t H16 = H / 8;
    const uint32_t rows_per_wg = H16 >= 512 ? 1u : 512u / H16;
    uint32_t chunks = 0;
    for (int i = 0; i < g.n; ++i)
        chunks = std::max(chunks, ((uint32_t)(group_tok(g, i + 1) - group_tok(g, i)) * k + rows_per_wg - 1) /
                                      rows_per_wg);
    const uint32_t rounds = (g.n + kXcds - 1) / kXcds;
    std::vector<char> seen(R, 0);
    for (uint32_t b = 0; b < rounds * kXcds * chunks; ++b) {
        const uint32_t m = b / kXcds;
        const int gi = (int)(m / chunks) * kXcds + (int)(b % kXcds);
        if (gi >= g.n) continue;
        const uint32_t first = (m % chunks) * rows_per_wg;
        const uint32_t n = (uint32_t)(group_tok(g, gi + 1) - group_tok(g, gi)) * k;
        for (uint32_t r = first; r < std::min(n, first + rows_per_wg); ++r) {
            const long p = (long)group_tok(g, gi) * k + r;
            if (seen[p]) fail("expand row copied twice", T, gi, p);
            seen[p] = 1;
        }
    }
    for (long p = 0; p < R; ++p)
        if (!seen[p]) fail("expand row never copied", T, k, p);
}

int main() {
    long cases = 0;
    for (int E : {1, 3, 8, 17, 64, 128, 256, 300, 512})
        for (int T : {1, 15, 16, 17, 63, 64, 65, 100, 255, 256, 257, 1000, 1023, 4096, 8192, 70000})
            for (int H : {8, 256, 2048, 7168}) {
                check_groups(T, E, H);
                ++cases;
            }
    const struct { int T, E, k, H; } lists[] = {{65, 128, 8, 2048}, {100, 17, 5, 8},   {300, 64, 6, 256},
                                                {1023, 64, 6, 4096}, {4096, 128, 8, 2048}, {257, 256, 8, 7168},
                                                {77, 8, 2, 264},    {5000, 3, 3, 8},    {129, 512, 16, 264},
                                                {8192, 256, 8, 7168}, {999, 33, 4, 64}};
    unsigned seed = 1;
    for (const auto& c : lists) {
        check_list(c.T, c.E, c.k, c.H, seed++);
        ++cases;
    }
    // workspace: the byte matrix of the two-launch form fits the int32 form's size
    for (int E = 1; E <= 512; ++E)
        for (int T : {1, 100, 4096, 65535}) {
            const int tb = route_tokens_per_block(E);
            const size_t nb = (T + tb - 1) / tb;
            if (nb * route_byte_row_vectors(E) * 16 > route_histogram_bytes(T, E)) fail("workspace", T, E, 0);
        }
    std::printf("ok %ld cases\n", cases);
    return 0;
}
