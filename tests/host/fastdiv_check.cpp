// Host check of the fast division used by the streaming kernels: for many
// divisors d and dividends n < 2^31, fastdiv(n, make_fastdiv(d)) == n / d.
#include <cstdio>
#include <cstdlib>
#include <random>

#include "device_common.h"

int main() {
    std::mt19937_64 rng(12345);
    long checked = 0;
    auto check = [&](uint32_t n, uint32_t d, const moe::FastDiv& f) {
        const uint32_t q = moe::fastdiv(n, f);
        ++checked;
        if (q != n / d) {
            std::printf("FAIL n=%u d=%u got %u want %u\n", n, d, q, n / d);
            std::exit(1);
        }
    };
    for (uint32_t d = 1; d <= 5000; ++d) {
        const moe::FastDiv f = moe::make_fastdiv(d);
        for (uint32_t n = 0; n < 3 * d + 3; ++n) check(n, d, f);
        for (int i = 0; i < 200; ++i) check((uint32_t)(rng() & 0x7FFFFFFFu), d, f);
        for (uint32_t m = 1; m < 64; ++m) {  // around multiples near the top of the range
            const uint64_t top = (0x7FFFFFFFull / d) * d;
            for (int64_t delta = -2; delta <= 2; ++delta) {
                const int64_t n = (int64_t)top - (int64_t)(m - 1) * d + delta;
                if (n >= 0 && n < 0x80000000ll) check((uint32_t)n, d, f);
            }
        }
    }
    for (int i = 0; i < 200000; ++i) {
        const uint32_t d = (uint32_t)(rng() % 0x7FFFFFFFu) + 1;
        const moe::FastDiv f = moe::make_fastdiv(d);
        check((uint32_t)(rng() & 0x7FFFFFFFu), d, f);
        check(0x7FFFFFFFu, d, f);
        check(d - 1, d, f);
        check(d < 0x7FFFFFFFu ? d : 0, d, f);
    }
    std::printf("ok %ld\n", checked);
    return 0;
}
