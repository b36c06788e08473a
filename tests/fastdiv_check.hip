// Host-side check of fast_div() in fa_divide.h (the function the kernels
// call) against the C++ integer division: exhaustive for small divisors and
// dividends, every quotient boundary n = q d - 1, q d, q d + d - 1 for
// divisors up to 2^17, dividends next to 2^31 - 1, and seeded random pairs
// over the whole range. Prints one line per failure (at most 20) and exits
// non-zero if any fails.
#include <cstdint>
#include <cstdio>

#include "fa_divide.h"

using fa::fast_div;
using fa::FastDiv;
using fa::make_fastdiv;

static long long failures = 0, checked = 0;

static void check(int n, int d, FastDiv f) {
    ++checked;
    const int got = fast_div(n, f), want = n / d;
    if (got != want) {
        if (failures < 20) std::printf("fast_div(%d, %d) = %d, expected %d\n", n, d, got, want);
        ++failures;
    }
}

int main() {
    // Exhaustive: divisors 1..64, dividends 0..2^20.
    for (int d = 1; d <= 64; ++d) {
        const FastDiv f = make_fastdiv(d);
        for (int n = 0; n < (1 << 20); ++n) check(n, d, f);
    }
    // Quotient boundaries for divisors up to 2^17, and the top of the range.
    for (int d = 1; d <= (1 << 17); ++d) {
        const FastDiv f = make_fastdiv(d);
        for (long long q = 1; q * d < 0x7fffffffLL; q = q < 64 ? q + 1 : q * 3 + 1) {
            const long long n0 = q * d;
            check((int)(n0 - 1), d, f);
            check((int)n0, d, f);
            if (n0 + d - 1 <= 0x7fffffffLL) check((int)(n0 + d - 1), d, f);
        }
        for (int k = 0; k < 4; ++k) check(0x7fffffff - k, d, f);
    }
    // Seeded random pairs over [1, 2^31) x [0, 2^31) (SplitMix64 stream).
    uint64_t s = 0x9e3779b97f4a7c15ull;
    auto next = [&]() {
        uint64_t z = (s += 0x9e3779b97f4a7c15ull);
        z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
        z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
        return z ^ (z >> 31);
    };
    for (int i = 0; i < 2000000; ++i) {
        const uint64_t r = next();
        int d = (int)(r & 0x7fffffffu);
        if (d == 0) d = 1;
        if (i & 1) d >>= (int)((r >> 40) % 31);  // spread divisor sizes over all bit lengths
        if (d == 0) d = 1;
        const int n = (int)((r >> 32) & 0x7fffffffu);
        check(n, d, make_fastdiv(d));
    }
    std::printf("checked %lld pairs, %lld failures\n", checked, failures);
    if (failures == 0) std::printf("all properties hold\n");
    return failures == 0 ? 0 : 1;
}
