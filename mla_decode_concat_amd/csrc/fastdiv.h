// Division by a run-time constant via one 64-bit multiply and a shift.
//
// For a divisor d >= 1 and numerators n < 2^31: with l = ceil(log2 d) and
// m = ceil(2^(31 + l) / d), floor(n / d) = floor(m * n / 2^(31 + l)).
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994, Theorem 4.2 with N = 31: the condition
// 2^(N+l) <= m*d <= 2^(N+l) + 2^l holds because m*d - 2^(N+l) < d <= 2^l.)
// m < 2^32 and n < 2^31, so the product fits in 64 bits.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MLA_DQ_HD __host__ __device__
#else
#define MLA_DQ_HD
#endif

struct FastDiv31 {
    uint64_t mul;
    uint32_t shift;
    uint32_t div;
};

inline FastDiv31 make_fastdiv31(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint32_t s = 31 + l;
    const uint64_t num = uint64_t(1) << s;              // s <= 62 for d < 2^31
    const uint64_t m = (num + d - 1) / d;
    return FastDiv31{m, s, d};
}

MLA_DQ_HD inline uint32_t fastdiv31(uint32_t n, const FastDiv31& f) {
    return uint32_t((uint64_t(n) * f.mul) >> f.shift);
}
