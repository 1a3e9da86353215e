// FP8 (OCP E4M3FN) quantisation arithmetic of the FP8 pack, for the device
// and for the host checks that pin it (the FP8 dispatch of the
// EnflameTechnology/DeepEP README feature notes: per-1x128 scales, round_scale,
// UE8M0 scales, one per-tensor fp8_quant_scale).
//
// Every quantity here must equal what IEEE fp32 arithmetic gives for the
// definition: scale s = a' / 448 (or a power of two, or the caller's scale),
// code = E4M3FN(x / s) rounded to nearest even and saturated at +/-448.  The
// kernels avoid the long IEEE division sequence with the functions below; the
// host test compiles this header with g++ and checks each against IEEE
// division and the reference encoder over the domains stated here.
#pragma once

#include <stdint.h>
#include <string.h>

#if defined(__HIPCC__)
#define MOEDX_FP8_HD __host__ __device__ __forceinline__
#else
#define MOEDX_FP8_HD inline
#endif

namespace moedx {

MOEDX_FP8_HD uint32_t fp8_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}
MOEDX_FP8_HD float fp8_float(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

// Nearest OCP E4M3FN code of q, ties to even, saturating at +/-448 (code
// 0x7E); NaN -> 0x7F; the sign of zero is kept.  Normal range (|q| >= 2^-6):
// round the fp32 significand to 3 bits with the round-half-even bias and
// re-bias the exponent from 127 to 7; subnormal range: the code is
// round-half-even(|q| * 2^9), exact in fp32 (a multiply by a power of two and
// a round to an integer).  Both ranges are computed and one is selected.
MOEDX_FP8_HD uint32_t e4m3_code(float q) {
    const uint32_t u = fp8_bits(q);
    const uint32_t mag = u & 0x7fffffffu;
    const uint32_t rn = (mag + 0x7ffffu + ((mag >> 20) & 1u)) >> 20;
    const uint32_t d = rn - (120u << 3);                 // wraps (unused) below 2^-6
    const uint32_t cn = d < 0x7eu ? d : 0x7eu;
    const uint32_t cs = (uint32_t)__builtin_rintf(fp8_float(mag) * 512.0f);
    const uint32_t c = (mag >= 0x3c800000u ? cn : cs) | ((u >> 24) & 0x80u);
    return mag > 0x7f800000u ? 0x7fu : c;
}

// a / s from rs = RN(1 / s), by the remainder correction of P. W. Markstein
// ("Computation of elementary functions on the IBM RISC System/6000
// processor", IBM J. Res. Develop. 34(1), 1990): q0 = RN(a * rs) is within an
// ulp of a / s, so the remainder r = a - q0 * s is exact under one fused
// multiply-add, and RN(q0 + r * rs) is the correctly rounded quotient.
// Domain where the result equals IEEE a / s (checked on the host for every
// fp32 divisor significand and every bf16 numerator significand, which covers
// every exponent pair by scaling): a, s, rs and the quotient normal, and
// a >= 2^-100 so that the remainder cannot underflow.
MOEDX_FP8_HD float quotient(float a, float s, float rs) {
    const float q0 = a * rs;
    const float r = __builtin_fmaf(-q0, s, a);
    return __builtin_fmaf(r, rs, q0);
}

// |x| / s clamped to 448 for one caller scale s in [2^-126, 2^126) (rs =
// RN(1 / s)) and any finite bf16 magnitude a: E4M3FN of the result equals
// E4M3FN of the IEEE quotient, saturated.  A numerator below 2^-100 is scaled
// by 2^64 before the division and the quotient back by 2^-64 (both exact while
// the quotient is normal; below 2^-126 every code is 0 either way), so the
// remainder never underflows; a quotient past 2^30 saturates whatever its
// rounding.
MOEDX_FP8_HD float tensor_quotient(float a, float s, float rs) {
    const bool tiny = a < 0x1p-100f;
    const float an = tiny ? a * 0x1p64f : a;
    const float qn = quotient(an, s, rs);
    const float q = tiny ? qn * 0x1p-64f : qn;
    const float sat = a * rs < 0x1p30f ? q : 448.0f;
    return sat < 448.0f ? sat : 448.0f;
}

// The smallest power of two >= t, for a positive normal or infinite t (inf
// stays inf).  For t = RN(a' / 448) this is also the smallest power of two >=
// the real quotient: t is a power of two only when the real quotient is one
// (a' has at most 24 significant bits, so a' / 448 is a power of two only for
// a' = 7 * 2^k and lies far from one otherwise).
MOEDX_FP8_HD float pow2_ceil(float t) {
    const uint32_t b = fp8_bits(t);
    return fp8_float((b & 0x7fffffu) ? (b & 0x7f800000u) + 0x800000u : b);
}

// The reciprocal of a power of two s in [2^-126, 2^126]: its exponent flipped
// (exact).
MOEDX_FP8_HD float pow2_reciprocal(float s) { return fp8_float((254u << 23) - fp8_bits(s)); }

// The per-block scale s = max(amax, 1e-4) / 448 for a block whose largest
// magnitude has the bit pattern ab (a finite bf16 value widened to fp32):
// correctly rounded (a quotient of a bf16 numerator by 448).
constexpr float kFp8FloorScale = 1e-4f / 448.0f;
MOEDX_FP8_HD float fp8_block_scale(uint32_t ab) {
    return ab > fp8_bits(1e-4f) ? quotient(fp8_float(ab), 448.0f, 1.0f / 448.0f)
                                : kFp8FloorScale;
}

}  // namespace moedx
