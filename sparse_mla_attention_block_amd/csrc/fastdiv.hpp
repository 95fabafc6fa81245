// Division of non-negative integers below 2^31 by a divisor fixed at launch
// time, as one multiply-high, one add and one shift (the round-up method of
// Granlund and Montgomery, "Division by invariant integers using
// multiplication", 1994): with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1, n / d = (mulhi(n, m) + n) >> l for every
// n < 2^31 (mulhi(n, m) <= n, so the sum stays below 2^32).  The host
// computes (m, l) once per launch; a runtime 32-bit division would otherwise
// expand into some twenty instructions and a 64-bit one into a hundred.
#pragma once

#include <stdint.h>

namespace dsv4 {

struct FastDiv {
    uint32_t d;   // divisor, 1 <= d < 2^31
    uint32_t m;   // magic multiplier
    uint32_t l;   // shift, ceil(log2 d)
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t l = 0;
    while ((uint64_t(1) << l) < d) ++l;
    const uint64_t m = ((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

// n / f.d for 0 <= n < 2^31.
__host__ __device__ inline uint32_t fdiv(uint32_t n, const FastDiv& f) {
    const uint32_t hi = (uint32_t)(((uint64_t)n * f.m) >> 32);
    return (hi + n) >> f.l;
}

}  // namespace dsv4
