// Pins the FP8 pack's arithmetic (csrc/fp8_codec.h) on the host, built with
// g++ against IEEE fp32 division and the oracle's brute-force E4M3FN encoder:
//   1. quotient(a, s, RN(1/s)) == RN(a / s) for every fp32 divisor significand
//      and every bf16 numerator significand (2^30 pairs; every exponent pair
//      follows by exact scaling while nothing under- or overflows);
//   2. the per-block scale fp8_block_scale == RN(max(a, 1e-4) / 448) and its
//      power-of-two form == the oracle's round_scale, for every bf16 value;
//   3. tensor_quotient: E4M3FN of it == E4M3FN of the IEEE quotient for every
//      finite bf16 numerator at scales spread over [2^-126, 2^126), including
//      subnormal numerators over tiny scales;
//   4. e4m3_code == the oracle's encoder on a dense fp32 sweep and on windows
//      around every code value and every midpoint, both signs, inf and NaN.
// Prints "ok <checks>" and exits 0, or names the first failure and exits 1.
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

#include "fp8_codec.h"

extern "C" {
uint8_t oracle_e4m3_encode(float v);
float oracle_pow2_scale(float ap);
}

using moedx::fp8_bits;
using moedx::fp8_float;

static std::atomic<uint64_t> g_checks{0};
static std::atomic<int> g_fail{0};

template <typename F>
static void parallel(int n, F f) {
    std::vector<std::thread> th;
    const int nt = (int)std::max(1u, std::thread::hardware_concurrency());
    for (int w = 0; w < nt; ++w)
        th.emplace_back([&, w] {
            for (int i = w; i < n && !g_fail.load(); i += nt) f(i);
        });
    for (auto& t : th) t.join();
}

static void fail(const char* what, uint32_t a, uint32_t b, uint32_t got, uint32_t want) {
    if (g_fail.exchange(1) == 0)
        std::printf("FAIL %s: a=0x%08x s=0x%08x got=0x%08x want=0x%08x\n", what, a, b, got, want);
}

// 1. Markstein quotient over every divisor significand x bf16 numerator significand.
static void check_quotient() {
    parallel(1 << 11, [](int chunk) {
        uint64_t n = 0;
        for (uint32_t lo = 0; lo < (1u << 12); ++lo) {
            const uint32_t sb = 0x3f800000u | ((uint32_t)chunk << 12) | lo;
            const float s = fp8_float(sb);
            const float rs = 1.0f / s;
            for (uint32_t m = 0; m < 128; ++m) {
                const float a = fp8_float(0x3f800000u | (m << 16));
                const float got = moedx::quotient(a, s, rs);
                const float want = a / s;
                if (fp8_bits(got) != fp8_bits(want)) fail("quotient", fp8_bits(a), sb, fp8_bits(got), fp8_bits(want));
                ++n;
            }
        }
        g_checks += n;
    });
}

// 2. Block scales: amax / 448 and its power-of-two ceiling, every bf16 magnitude.
static void check_block_scales() {
    for (uint32_t h = 0; h < 0x7f80u; ++h) {  // every finite non-negative bf16
        const uint32_t ab = h << 16;
        const float a = fp8_float(ab);
        const float ap = a > 1e-4f ? a : 1e-4f;
        const float s = moedx::fp8_block_scale(ab);
        const float want = ap / 448.0f;
        if (fp8_bits(s) != fp8_bits(want)) fail("block scale", ab, 0, fp8_bits(s), fp8_bits(want));
        const float p = moedx::pow2_ceil(s);
        const float pw = oracle_pow2_scale(ap);
        if (fp8_bits(p) != fp8_bits(pw)) fail("pow2 scale", ab, 0, fp8_bits(p), fp8_bits(pw));
        const float rp = moedx::pow2_reciprocal(p);
        if (fp8_bits(rp) != fp8_bits(1.0f / p)) fail("pow2 reciprocal", ab, 0, fp8_bits(rp), fp8_bits(1.0f / p));
        g_checks += 3;
    }
    if (fp8_bits(moedx::pow2_ceil(INFINITY)) != fp8_bits(INFINITY)) fail("pow2 inf", 0, 0, 0, 0);
}

// 3. The per-tensor quotient: codes against the IEEE quotient's codes.
static void check_tensor() {
    std::vector<uint32_t> scales;
    uint32_t seed = 12345u;
    auto rnd = [&] { seed = seed * 1664525u + 1013904223u; return seed; };
    for (int e = -126; e <= 125; ++e) {
        const uint32_t ebits = (uint32_t)(e + 127) << 23;
        for (uint32_t m : {0u, 1u, 0x7fffffu, 0x400000u, 0x34b4b4u})
            scales.push_back(ebits | m);
        for (int i = 0; i < 3; ++i) scales.push_back(ebits | (rnd() & 0x7fffffu));
    }
    for (float f : {0x1p-120f, 0x1p-20f, 0.37f, 1e3f, 0x1p120f, 0.0123f, 0.5f, 1.0f / 448.0f})
        scales.push_back(fp8_bits(f));
    scales.push_back(0x00b4b4b4u + 0x00800000u);  // just above 2^-126
    parallel((int)scales.size(), [&](int i) {
        const float s = fp8_float(scales[i]);
        if (!(s >= 0x1p-126f && s < 0x1p126f)) return;
        const float rs = 1.0f / s;
        uint64_t n = 0;
        for (uint32_t h = 0; h < 0x7f80u; ++h) {  // every finite non-negative bf16
            const float a = fp8_float(h << 16);
            const uint32_t got = moedx::e4m3_code(moedx::tensor_quotient(a, s, rs));
            const uint32_t want = moedx::e4m3_code(a / s);
            if (got != want) fail("tensor quotient code", h << 16, scales[i], got, want);
            ++n;
        }
        g_checks += n;
    });
    // against the oracle's encoder itself on a subset of the scales
    parallel((int)scales.size() / 8, [&](int i) {
        const float s = fp8_float(scales[8 * i]);
        const float rs = 1.0f / s;
        uint64_t n = 0;
        for (uint32_t h = 0; h < 0xff80u; h += 3) {
            if ((h & 0x7f80u) == 0x7f80u) continue;  // inf / NaN take another path
            const float x = fp8_float(h << 16);
            const float q = moedx::tensor_quotient(std::fabs(x), s, rs);
            const uint32_t got = moedx::e4m3_code(fp8_float(fp8_bits(q) | (fp8_bits(x) & 0x80000000u)));
            const uint32_t want = oracle_e4m3_encode(x / s);
            if (got != want) fail("tensor code vs oracle", h << 16, scales[8 * i], got, want);
            ++n;
        }
        g_checks += n;
    });
}

// 4. e4m3_code against the oracle's encoder.
static void check_encoder() {
    auto one = [](uint32_t u) {
        for (uint32_t sign : {0u, 0x80000000u}) {
            const float v = fp8_float(u | sign);
            const uint32_t got = moedx::e4m3_code(v);
            const uint32_t want = oracle_e4m3_encode(v);
            if (got != want) fail("e4m3_code", u | sign, 0, got, want);
        }
    };
    const uint32_t top = fp8_bits(1024.0f);
    const int parts = 64;
    parallel(parts, [&](int p) {
        uint64_t n = 0;
        for (uint32_t u = (uint32_t)p * 61u; u <= top; u += 61u * parts, n += 2) one(u);
        g_checks += n;
    });
    // windows around every code value and every midpoint between neighbours
    std::vector<uint32_t> centres;
    for (int c = 0; c <= 0x7e; ++c) {
        const float v = (c < 8) ? std::ldexp((float)c, -9)
                                : std::ldexp(1.0f + (float)(c & 7) / 8.0f, (c >> 3) - 7);
        centres.push_back(fp8_bits(v));
        if (c < 0x7e) {
            const float w = (c + 1 < 8) ? std::ldexp((float)(c + 1), -9)
                                        : std::ldexp(1.0f + (float)((c + 1) & 7) / 8.0f, ((c + 1) >> 3) - 7);
            centres.push_back(fp8_bits(0.5f * (v + w)));
        }
    }
    centres.push_back(fp8_bits(464.0f));  // midpoint of 448 and the next step up
    parallel((int)centres.size(), [&](int i) {
        const uint32_t c = centres[i];
        const uint32_t lo = c > 4096u ? c - 4096u : 0u;
        for (uint32_t u = lo; u <= c + 4096u; ++u) one(u);
        g_checks += 2 * (c + 4097u - lo);
    });
    for (uint32_t u : {0x7f800000u, 0x7f800001u, 0x7fc00000u, 0x7fffffffu, fp8_bits(3.0e38f)}) one(u);
}

int main() {
    check_block_scales();
    check_encoder();
    check_tensor();
    check_quotient();
    if (g_fail.load()) return 1;
    std::printf("ok %llu\n", (unsigned long long)g_checks.load());
    return 0;
}
