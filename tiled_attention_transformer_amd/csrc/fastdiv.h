// Division of a non-negative 31-bit numerator by a divisor that is fixed for
// a launch, as one multiply-high, an add and a shift (the round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", PLDI 1994): with s = ceil(log2 d) and
// m = floor(2^32 (2^s - d) / d) + 1, for every 0 <= n < 2^31
//   n / d = (mulhi32(n, m) + n) >> s
// (m + 2^32 is ceil(2^(32+s) / d), whose excess over 2^(32+s) / d is at most
// 1, so the quotient is exact below 2^32; below 2^31 the sum fits 32 bits).
// The kernels' item decode divides by head and batch counts at every item
// change; a runtime integer division there is a chain through the vector
// unit's reciprocal, this is three scalar instructions.
#pragma once
#include <stdint.h>

namespace attn {

struct FastDiv {
    uint32_t m, s;
};

// host: the constants for a divisor 1 <= d < 2^31
inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
    return FastDiv{(uint32_t)m, s};
}

// the quotient as the kernels compute it (host form, for the tests)
inline uint32_t fastdiv_apply(uint32_t n, FastDiv f) {
    return (uint32_t)((((uint64_t)n * f.m) >> 32) + n) >> f.s;
}

}  // namespace attn
