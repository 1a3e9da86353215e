// Division of a non-negative 32-bit index by a launch constant, as one
// multiply-high and a shift (the integer division it replaces is a few dozen
// scalar instructions per wave).
//
// For a divisor d >= 1 let s = ceil(log2 d) and mul = ceil(2^(31+s) / d), so
// mul * d = 2^(31+s) + e with 0 <= e < d <= 2^s.  Then for 0 <= n < 2^31,
//   n * mul / 2^(31+s) = n / d + n * e / (d * 2^(31+s)),
// and the second term is below 1/d because n * e < 2^31 * 2^s; the floor is
// therefore floor(n / d) exactly.  mul < 2^32 since d > 2^(s-1).
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MOEDX_HD __host__ __device__
#else
#define MOEDX_HD
#endif

namespace moedx {

struct FastDiv {
    uint32_t mul;
    uint32_t shift;
    uint32_t d;
    MOEDX_HD inline uint32_t div(uint32_t n) const {
        return (uint32_t)(((uint64_t)n * mul) >> shift);
    }
};

inline FastDiv make_fastdiv(uint32_t d) {
    uint32_t s = 0;
    while (((uint64_t)1 << s) < d) ++s;
    const uint64_t mul = ((((uint64_t)1) << (31 + s)) + d - 1) / d;
    return FastDiv{(uint32_t)mul, 31 + s, d};
}

}  // namespace moedx
