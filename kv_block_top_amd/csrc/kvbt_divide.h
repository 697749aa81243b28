// kvbt_divide.h -- division by a divisor fixed for a launch (the heads per row, the
// decode query length), taken by the kernels as one multiply and one shift instead of
// the division sequence the compiler emits for a run-time divisor. Plain C++ (constexpr
// functions are usable on both sides), so the host test checks the same code.
#pragma once

#include <stdint.h>

namespace kvbt {

// For a divisor d >= 1 and l = ceil(log2 d), m = ceil(2^(31 + l) / d) gives
// floor(n / d) = floor(n m / 2^(31 + l)) for every 0 <= n < 2^31: Granlund and
// Montgomery, "Division by invariant integers using multiplication" (PLDI 1994),
// Theorem 4.2 with N = 31, whose condition 2^(N+l) <= m d <= 2^(N+l) + 2^l holds because
// m d - 2^(N+l) < d <= 2^l. m stays below 2^32 for every d < 2^31, and n m below 2^63.
struct Divisor {
    uint32_t mul;
    uint32_t shift;
};

constexpr Divisor make_divisor(uint32_t d)
{
    uint32_t l = 0;
    while ((uint64_t{1} << l) < d) ++l;
    return Divisor{(uint32_t)(((uint64_t{1} << (31 + l)) + d - 1) / d), 31 + l};
}

// floor(n / d) for 0 <= n < 2^31, from make_divisor(d)'s fields.
constexpr uint32_t divide_by(uint32_t n, uint32_t mul, uint32_t shift)
{
    return (uint32_t)(((uint64_t)n * mul) >> shift);
}

}  // namespace kvbt
