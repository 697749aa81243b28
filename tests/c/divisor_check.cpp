// divisor_check.cpp -- the kernels' division by a launch-fixed divisor (kvbt_divide.h)
// against the exact quotient, on the host (the same constexpr code the kernels run).
// Divisors 1..4096 exhaustively over dividends 0..2^16 and around every multiple of d
// near the top of the range, plus every power of two and its neighbours, and a seeded
// sample of divisors up to 2^31 - 1. Built and run by tests/test_c_abi.py.
#include <stdint.h>
#include <stdio.h>

#include <initializer_list>

#include "kvbt_divide.h"

static long failures = 0;

static void check(uint32_t d, uint32_t n)
{
    const kvbt::Divisor v = kvbt::make_divisor(d);
    const uint32_t got = kvbt::divide_by(n, v.mul, v.shift);
    if (got != n / d) {
        if (failures < 10) fprintf(stderr, "d %u n %u: %u, want %u\n", d, n, got, n / d);
        ++failures;
    }
}

static void check_divisor(uint32_t d)
{
    const uint32_t top = 0x7FFFFFFFu;   // largest dividend (row and pair indices < 2^31)
    for (uint32_t n = 0; n <= 4096; ++n) check(d, n);
    check(d, top);
    // around the last multiples of d below 2^31, and around 2^31 / 2, 2^31 / 4
    for (uint32_t base : {top, top / 2, top / 4, top / 3}) {
        const uint32_t k = base / d;
        for (int j = -2; j <= 0; ++j) {
            const int64_t m = ((int64_t)k + j) * d;
            for (int e = -1; e <= 1; ++e) {
                const int64_t n = m + e;
                if (n >= 0 && n <= top) check(d, (uint32_t)n);
            }
        }
    }
}

int main()
{
    for (uint32_t d = 1; d <= 4096; ++d) {
        check_divisor(d);
        if (d <= 64)
            for (uint32_t n = 0; n <= (1u << 16); ++n) check(d, n);
    }
    for (int s = 12; s <= 30; ++s)
        for (int e = -1; e <= 1; ++e) check_divisor((1u << s) + e);
    check_divisor(0x7FFFFFFFu);
    uint64_t x = 0x9E3779B97F4A7C15ull;   // splitmix-style sample of large divisors
    for (int i = 0; i < 20000; ++i) {
        x += 0x9E3779B97F4A7C15ull;
        uint64_t z = x;
        z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
        z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
        z ^= z >> 31;
        const uint32_t d = (uint32_t)(z % 0x7FFFFFFFu) + 1;
        check_divisor(d);
    }
    if (failures) {
        fprintf(stderr, "%ld wrong quotients\n", failures);
        return 1;
    }
    printf("divisor checks passed\n");
    return 0;
}
