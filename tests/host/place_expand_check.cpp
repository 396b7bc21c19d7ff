// Host check of the placing destination-order expand (place_expand.hip):
// a model of every workgroup's index arithmetic for random routings, with
// the launch shape from place_expand_shape.  It checks that
//  * every LDS and global index the kernel forms stays in bounds: group slots
//    <= kPeSlotsPerLane * 1024, bitmap words <= kPeMaskWordsMax, slice rows
//    < kPeRowsMax, source prefetch inside the group, histogram rows < nb;
//  * every group's rows are cut into chunks dealt to the workgroups so that
//    each destination position is placed and copied exactly once;
//  * each row, found back from its position as the kernel does (expert by
//    the group's count prefix, bitmap word by its popcount prefix, token by
//    select_bit, slot by the token's ids), is the slot the stable counting
//    sort puts there.
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

static void check(int T, int E, int k, int H, int pad, int wpg, unsigned seed) {
    const PlaceExpandShape sh = place_expand_shape(T, E, k, H, wpg);
    if (!sh.ok) {
        // outside the path: only allowed past its documented limits
        if (T <= kRouteTwoPassMaxTokens && route_byte_row_vectors(E) <= 16 && H < (1 << 24))
            fail("shape refused", T, E, H);
        return;
    }
    const RowGroups& g = sh.groups;
    const int tb = route_tokens_per_block(E);
    const int nb = (T + tb - 1) / tb;
    if (g.n % kXcds != 0 || g.n > kXcds * kMaxGroupsPerXcd) fail("group count", T, E, g.n);
    if (group_row(g, g.n) != nb || group_tok(g, g.n) != T) fail("group ends", T, E, g.n);
    if (sh.Rc < 1 || sh.Rc > (uint32_t)kPeRowsMax) fail("chunk rows", T, H, sh.Rc);
    if (sh.grid != (uint32_t)((g.n + kXcds - 1) / kXcds) * kXcds * sh.S) fail("grid", T, sh.grid, sh.S);
    // random routing: k distinct experts per token
    std::mt19937 rng(seed);
    std::vector<int> ids((size_t)T * k), perm(E);
    for (int t = 0; t < T; ++t) {
        for (int e = 0; e < E; ++e) perm[e] = e;
        std::shuffle(perm.begin(), perm.end(), rng);
        for (int j = 0; j < k; ++j) ids[(size_t)t * k + j] = perm[j];
    }
    // the route's answer: stable counting sort, segments padded to pad
    std::vector<long> cnt(E, 0), off(E + 1, 0), cur(E);
    for (int id : ids) ++cnt[id];
    for (int e = 0; e < E; ++e) off[e + 1] = off[e] + (cnt[e] + pad - 1) / pad * pad;
    std::vector<long> want((size_t)T * k);
    for (int e = 0; e < E; ++e) cur[e] = off[e];
    for (size_t s = 0; s < ids.size(); ++s) want[s] = cur[ids[s]]++;
    std::vector<int> placed((size_t)T * k, 0), copied((size_t)T * k, 0);
    const uint32_t H16 = (uint32_t)H / 8;
    // every workgroup of the grid
    for (uint32_t b = 0; b < sh.grid; ++b) {
        const uint32_t m = b / kXcds;
        const int gi = (int)(m / sh.S) * kXcds + (int)(b % kXcds);
        const uint32_t c = m % sh.S;
        if (gi >= g.n) fail("group index", T, b, gi);
        const int gt0 = group_tok(g, gi), gt1 = group_tok(g, gi + 1), gr0 = group_row(g, gi);
        if (gr0 > nb || gt0 != std::min(T, gr0 * tb)) fail("group start", T, gi, gr0);
        const int ntok = gt1 - gt0, nslot = ntok * k;
        const int W = (ntok + 63) / 64;
        if (nslot > kPeSlotsPerLane * 1024) fail("group slots", T, gi, nslot);
        if (E * W > kPeMaskWordsMax) fail("bitmap words", T, gi, E * W);
        const uint32_t src_n = (uint32_t)ntok * H16, per = (src_n + sh.S - 1) / sh.S;
        // the prefetch loads j in [c * per, min(src_n, c * per + per)): inside the
        // group's source whenever the 32-bit products do not wrap
        if ((uint64_t)c * per + per >= (1ull << 32)) fail("prefetch range", T, gi, c);
        // the group's counts and bitmaps, then every row of this workgroup
        // found back as the kernel does it: expert by the group's prefix,
        // word by the bitmap word prefix, token by select_bit, slot by id
        std::vector<long> gcnt(E, 0), gcum(E + 1, 0), base(E, 0);
        std::vector<unsigned long long> masks((size_t)E * W, 0ull);
        for (int s = 0; s < nslot; ++s) {
            const int e = ids[(size_t)gt0 * k + s];
            ++gcnt[e];
            masks[(size_t)e * W + (s / k) / 64] |= 1ull << ((s / k) % 64);
        }
        for (int e = 0; e < E; ++e) gcum[e + 1] = gcum[e] + gcnt[e];
        for (size_t s = 0; s < (size_t)gt0 * k; ++s) ++base[ids[s]];
        std::vector<int> pcw((size_t)E * W, 0);
        for (int e = 0; e < E; ++e)
            for (int w = 1; w < W; ++w)
                pcw[(size_t)e * W + w] = pcw[(size_t)e * W + w - 1] + __builtin_popcountll(masks[(size_t)e * W + w - 1]);
        const uint32_t nchunks = ((uint32_t)nslot + sh.Rc - 1) / sh.Rc;
        const uint32_t mine = nchunks > c ? (nchunks - c + sh.S - 1) / sh.S : 0u;
        uint32_t rows = mine * sh.Rc;
        if (mine > 0 && (c + (mine - 1) * sh.S + 1) * sh.Rc > (uint32_t)nslot)
            rows -= (c + (mine - 1) * sh.S + 1) * sh.Rc - (uint32_t)nslot;
        if (rows > (uint32_t)kPeRowsMax) fail("slice rows", T, b, rows);
        if ((uint64_t)rows * H16 >= (1ull << 31)) fail("items", T, b, rows);
        for (uint32_t i = 0; i < rows; ++i) {
            const uint32_t p = (c + sh.S * (i / sh.Rc)) * sh.Rc + i % sh.Rc;
            if (p >= (uint32_t)nslot) fail("position", T, b, p);
            int lo = 0, hi = E;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if ((uint32_t)gcum[mid] <= p) lo = mid; else hi = mid;
            }
            const int e = lo;
            const int rank = (int)p - (int)gcum[e];
            if (rank < 0 || rank >= gcnt[e]) fail("rank", T, e, rank);
            int wl = 0, wh = W;
            while (wh - wl > 1) {
                const int mid = (wl + wh) >> 1;
                if (pcw[(size_t)e * W + mid] <= rank) wl = mid; else wh = mid;
            }
            const unsigned long long mw = masks[(size_t)e * W + wl];
            const int r2 = rank - pcw[(size_t)e * W + wl];
            if (r2 < 0 || r2 >= __builtin_popcountll(mw)) fail("word", T, e, r2);
            const int tl = wl * 64 + select_bit(mw, r2);
            if (tl >= ntok || !((mw >> (tl % 64)) & 1ull)) fail("select", T, e, tl);
            int j = 0;
            while (j < k - 1 && ids[(size_t)(gt0 + tl) * k + j] != e) ++j;
            if (ids[(size_t)(gt0 + tl) * k + j] != e) fail("slot id", T, tl, e);
            const size_t gs = (size_t)(gt0 + tl) * k + j;
            const long d = off[e] + base[e] + rank;
            if (d != want[gs]) fail("destination", T, (long)gs, d);
            if (d < 0 || d >= off[E]) fail("copied row", T, b, d);
            ++placed[gs];
            ++copied[gs];
        }
    }
    for (size_t s = 0; s < placed.size(); ++s) {
        if (placed[s] != 1) fail("slot placed", T, (long)s, placed[s]);
        if (copied[s] != 1) fail("slot copied", T, (long)s, copied[s]);
    }
}

int main() {
    const int shapes[][4] = {{4096, 128, 8, 2048}, {1500, 96, 6, 256}, {3000, 64, 6, 8},   {777, 256, 8, 16392},
                             {5000, 16, 4, 520},   {2500, 128, 8, 1024}, {4100, 200, 6, 264}, {8192, 256, 8, 7168},
                             {1023, 64, 6, 4096},  {65, 8, 2, 16},       {300, 3, 3, 8},      {20000, 64, 2, 64},
                             {300, 16, 4, 32768},  {65, 128, 8, 2048},   {65535, 8, 2, 16},   {9000, 300, 4, 64},
                             {70000, 64, 2, 64}};
    const int wpgs[] = {0, 1, 2, 7, 64, 300};
    unsigned seed = 1;
    for (const auto& sh : shapes)
        for (int wpg : wpgs)
            for (int pad : {1, 7, 128}) check(sh[0], sh[1], sh[2], sh[3], pad, wpg, seed++);
    std::printf("ok\n");
    return 0;
}
