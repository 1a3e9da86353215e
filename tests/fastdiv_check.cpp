// Checks FastDiv against the integer division it replaces, for every divisor
// in [1, 4096] and some large ones: all n below 4096, the last 4096 values
// below 2^31, and n = k d - 1, k d, k d + 1 for sampled k and the last 64 k.
#include <cstdint>
#include <cstdio>
#include <vector>

#include "fastdiv.h"

int main() {
    std::vector<uint32_t> divisors;
    for (uint32_t d = 1; d <= 4096; ++d) divisors.push_back(d);
    for (uint32_t d : {65535u, 65536u, 65537u, 1000003u, (1u << 20) + 1, (1u << 30) - 1, 1u << 30,
                       (1u << 31) - 1})
        divisors.push_back(d);
    const uint64_t top = 1ull << 31;
    uint64_t checked = 0;
    for (uint32_t d : divisors) {
        const moedx::FastDiv f = moedx::make_fastdiv(d);
        auto ok = [&](uint64_t n) {
            if (n >= top) return true;
            ++checked;
            if (f.div((uint32_t)n) == (uint32_t)(n / d)) return true;
            std::printf("FAIL d=%u n=%llu\n", d, (unsigned long long)n);
            return false;
        };
        for (uint64_t n = 0; n < 4096; ++n)
            if (!ok(n)) return 1;
        for (uint64_t n = top - 4096; n < top; ++n)
            if (!ok(n)) return 1;
        const uint64_t kmax = (top - 1) / d;
        const uint64_t step = kmax > 20000 ? kmax / 20000 : 1;
        for (uint64_t k = 1; k <= kmax + 1; k += step)
            if (!ok(k * d - 1) || !ok(k * d) || !ok(k * d + 1)) return 1;
        for (uint64_t k = kmax > 64 ? kmax - 64 : 1; k <= kmax + 1; ++k)
            if (!ok(k * d - 1) || !ok(k * d) || !ok(k * d + 1)) return 1;
    }
    std::printf("ok %llu\n", (unsigned long long)checked);
    return 0;
}
