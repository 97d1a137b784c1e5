// OCP e4m3 and bf16 conversions in integer arithmetic, for gfx950 kernels.
//
// The pages only say FP8; the format taken is OCP e4m3 (bias 7, largest finite
// 448, NaN at S.1111.111, subnormals), rounding to nearest with ties to even and
// saturating at 448.  Written in integer operations on the float32 bit pattern so
// that rounding does not depend on the conversion instructions' modes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>

namespace moe {

constexpr float kE4M3Max = 448.0f;

// Bit casts usable on both sides, so the host can run the same codec in tests.
__host__ __device__ __forceinline__ uint32_t f2u(float f) { return __builtin_bit_cast(uint32_t, f); }
__host__ __device__ __forceinline__ float u2f(uint32_t u) { return __builtin_bit_cast(float, u); }

// Encode |v| (float32) to an e4m3 code, sign from v.  `hint` tells in which
// direction the exact value lies relative to v when v is the rounded result of
// a division: +1 larger magnitude, -1 smaller, 0 exact.  It only matters when
// v sits exactly on a midpoint between two codes.
__host__ __device__ __forceinline__ uint32_t e4m3_encode(float v, int hint) {
    const uint32_t bits = f2u(v);
    const uint32_t sign = (bits >> 24) & 0x80u;
    const uint32_t mag = bits & 0x7FFFFFFFu;
    const uint32_t fexp = mag >> 23;  // biased float32 exponent
    // normal e4m3 (|v| >= 2**-6): keep 3 mantissa bits, round on the 20 below
    const uint32_t rem = mag & 0xFFFFFu;
    uint32_t cn = ((fexp - 120u) << 3) | ((mag >> 20) & 7u);
    cn += (rem > 0x80000u || (rem == 0x80000u && (hint > 0 || (hint == 0 && (cn & 1u))))) ? 1u : 0u;
    // subnormal e4m3: value = k * 2**-9 with k = round(|v| * 512) in 0..8
    const float t = u2f(mag) * 512.0f;  // exact scaling by 2**9
    const float fl = floorf(t);
    const float frac = t - fl;                      // exact
    uint32_t cs = (uint32_t)fl;                     // k == 8 is code 0x08 = 2**-6
    cs += (frac > 0.5f || (frac == 0.5f && (hint > 0 || (hint == 0 && (cs & 1u))))) ? 1u : 0u;
    uint32_t code = fexp >= 121u ? cn : cs;         // a carry of cn moves into the exponent
    code = mag >= 0x43E00000u ? 0x7Eu : code;       // >= 448 (and inf): saturate
    code |= sign;
    return mag > 0x7F800000u ? 0x7Fu : code;        // NaN
}

// Quotient v / s rounded once to e4m3: the float32 quotient plus the sign of the
// exact remainder, so the result equals rounding the exact rational quotient.
__host__ __device__ __forceinline__ uint32_t e4m3_encode_div(float v, float s) {
    const float q = v / s;                          // IEEE division, round to nearest
    const float r = fmaf(-q, s, v);                 // exact remainder v - q*s
    const int hint = (r == 0.0f) ? 0 : (((r > 0.0f) == (q > 0.0f)) ? 1 : -1);
    return e4m3_encode(q, hint);
}

// A bracket of the exact quotient v / s from products with a moved reciprocal: the lower end
// fp32(v * rlo), the upper fp32(v * rhi), rlo = fp32(r (1 - 2^-21)), rhi = fp32(r (1 + 2^-21)),
// r = fp32(1 / s).  Three roundings of 2^-24 each (r, the moved reciprocal, the product) keep
// each end on its side of the exact quotient, by at least 5 * 2^-24 relative, and less than
// 2^-20 from it.  Quotients below float32's normal range (where the relative bound fails) round
// to code 0 at either end and exactly.  The conversion (round to nearest even, OCP e4m3) takes
// the signed ends: a code's sign is its value's, zeros and values that round to zero included.
constexpr float kBracketLo = 1.0f - 0x1p-21f;  // (exact in float32)
constexpr float kBracketHi = 1.0f + 0x1p-21f;

// e4m3 codes of v0 / s and v1 / s (low byte: v0) with r = fp32(1 / s), s >= kTinyScale, or
// kQuantExact when the pair needs the exact path (e4m3_encode_div): the codes of the
// bracket's two ends, which are the code of the exact quotient when they agree; otherwise a
// rounding midpoint lies in the bracket (about 4 in 2**20 values).  SAT: quotients may exceed
// 448 (a static scale); both ends are clamped to +-448 first, which the conversion keeps at
// 448.  Without SAT, |q| <= 448 (1 + 2**-22) holds by construction of the scale, and the upper
// end, below 448 (1 + 2**-20), still converts to 448.
constexpr uint32_t kQuantExact = 0xFFFFFFFFu;
constexpr uint32_t kE4M3MaxBits = 0x43E00000u;  // 448.0f

template <bool SAT = false>
__device__ __forceinline__ uint32_t e4m3_quant2_fast(float v0, float v1, float r) {
    const float rlo = r * kBracketLo, rhi = r * kBracketHi;  // (per row: hoisted by the compiler)
    float l0 = v0 * rlo, l1 = v1 * rlo, h0 = v0 * rhi, h1 = v1 * rhi;
    if (SAT) {
        l0 = __builtin_amdgcn_fmed3f(l0, -kE4M3Max, kE4M3Max);
        l1 = __builtin_amdgcn_fmed3f(l1, -kE4M3Max, kE4M3Max);
        h0 = __builtin_amdgcn_fmed3f(h0, -kE4M3Max, kE4M3Max);
        h1 = __builtin_amdgcn_fmed3f(h1, -kE4M3Max, kE4M3Max);
    }
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(l0, l1, 0, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(h0, h1, 0, false);
    return ((lo ^ hi) & 0xFFFFu) == 0u ? (lo & 0xFFFFu) : kQuantExact;
}

__host__ __device__ __forceinline__ float e4m3_decode(uint32_t c) {
    const uint32_t e = (c >> 3) & 15u, m = c & 7u;
    float mag;
    if (e == 15u && m == 7u) return u2f(0x7FC00000u);
    if (e == 0u) mag = (float)m * 0.001953125f;                  // m * 2**-9
    else mag = u2f(((e + 120u) << 23) | (m << 20));  // (1+m/8) * 2**(e-7)
    return (c & 0x80u) ? -mag : mag;
}

// Magnitude code of |v| / s from the codes lo <= hi that the conversion gives for the two
// ends of the bracket around the float32 estimate.  When they differ, the rounding midpoint
// m between the two adjacent codes' values (exact in float32) lies in the bracket, and
// the exact quotient is above, below or on it as |v| - m s is positive, negative or zero:
// one fused multiply-add computes that difference with a single rounding, which keeps
// its sign and gives zero only for an exact zero.  On the midpoint the even code wins.
// The midpoint above code lo (0..0x7D) is its value with one more mantissa bit: for a
// normal code the float32 bits of (1 + m/8 + 1/16) 2^(e-7), for a subnormal (2m + 1) 2^-10.
// Equal ends give that code whatever the sign.  Both midpoint forms are computed and every
// choice is a select: per-element branches cost more than the arithmetic, since a wave
// takes the union of its lanes' paths.
__device__ __forceinline__ uint32_t e4m3_pick(float v, float s, uint32_t lo, uint32_t hi) {
    const uint32_t e = lo >> 3, m = lo & 7u;
    const float normal = u2f(((e + 120u) << 23) | (m << 20) | (1u << 19));
    const float sub = (float)(2u * m + 1u) * 0.0009765625f;  // 2^-10
    const float mid = e != 0u ? normal : sub;
    const float d = fmaf(-mid, s, fabsf(v));
    const uint32_t off = d > 0.0f ? hi : lo;
    const uint32_t even = (lo & 1u) ? hi : lo;
    return d == 0.0f ? even : off;
}

// The codes of e4m3_quant2_fast, always resolved, saturating at 448: the same codes as
// rounding the exact quotients v / s, without a division.  Needs s >= kTinyScale (then
// r = fp32(1 / s) is finite and the bracket holds at most one midpoint, so its two ends
// are equal or adjacent codes; and |v| - m s, when not zero, is at least the smallest
// subnormal, so the fused multiply-add keeps its sign).  Smaller scales go through
// e4m3_quant2_tiny.  bf16 inputs over a scale with a short mantissa put many quotients on
// or next to a midpoint, so a token can send every value through here.
__device__ __forceinline__ uint32_t e4m3_quant2_exact(float v0, float v1, float s, float r) {
    const uint32_t a0 = min(f2u(v0 * r) & 0x7FFFFFFFu, kE4M3MaxBits);
    const uint32_t a1 = min(f2u(v1 * r) & 0x7FFFFFFFu, kE4M3MaxBits);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u2f(max(a0, 4u) - 4u), u2f(max(a1, 4u) - 4u), 0, false);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(u2f(a0 + 4u), u2f(a1 + 4u), 0, false);
    const uint32_t sign = ((f2u(v0) >> 24) & 0x80u) | ((f2u(v1) >> 16) & 0x8000u);
    const uint32_t c0 = e4m3_pick(v0, s, lo & 0xFFu, hi & 0xFFu);
    const uint32_t c1 = e4m3_pick(v1, s, (lo >> 8) & 0xFFu, (hi >> 8) & 0xFFu);
    return c0 | (c1 << 8) | sign;
}

// The codes of e4m3_quant2_fast, always resolved without the exact path, for bf16 values
// v over their row's scale s = fp32(amax / 448) >= kTinyScale, amax a bf16 value too.  Then the bracket's
// ends differ only at an exact tie of the ideal ratio: 448 v / amax and a midpoint m
// (5 significant bits) are ratios of small integers (v and amax carry 8-bit
// significands, 448 = 7 * 2^6), so if they differ, they differ by at least ~2^-17
// relative, far more than the bracket's ~2^-21.  At such a tie v / s = m amax / (448 s)
// lies on the side of m that the rounding of s gives, the same for the whole row: `dir`
// is the sign of amax - 448 s (one fused multiply-add, exact in sign): below m (< 0: the
// lower code), above (> 0: the upper), on it (0, s exact: the even code).
//
// Since dir is one sign for the whole row, only one end of the bracket is needed when it is
// not zero: the ends of e4m3_quant2_fast's bracket (products with a moved reciprocal) lie
// less than 2^-20 from the exact quotient, far inside the 2^-17 gap, so they differ only at
// an exact tie.

// Codes of 4 values (low byte: v0) at one end of the bracket: rq = rhi for dir > 0, rlo for
// dir < 0.
__device__ __forceinline__ uint32_t e4m3_quant4_bf16_end(float v0, float v1, float v2, float v3, float rq) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(v0 * rq, v1 * rq, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(v2 * rq, v3 * rq, lo, true);
}

// dir == 0 (s exact): both ends, and the even code of the two where they differ.
__device__ __forceinline__ uint32_t e4m3_quant4_bf16_even(float v0, float v1, float v2, float v3, float rlo,
                                                          float rhi) {
    const uint32_t lo = e4m3_quant4_bf16_end(v0, v1, v2, v3, rlo);
    const uint32_t hi = e4m3_quant4_bf16_end(v0, v1, v2, v3, rhi);
    const uint32_t odd = (lo & 0x01010101u) * 0xFFu;  // bytes whose lower code is odd
    return (hi & odd) | (lo & ~odd);
}

// Scales below kTinyScale: those of a row whose largest magnitude is below about
// 448 * 2^-96 (down to subnormal float32 scales, whose reciprocal overflows).  Such a
// scale and its values are first multiplied by kTinyLift: the quotients are unchanged
// (powers of two scale exactly, and the lifted values of a row stay far below the float32
// range), the lifted scale is a normal float32 of at least 2^-85, and 1 / s is finite.
constexpr float kTinyScale = 0x1p-96f;
constexpr float kTinyLift = 0x1p64f;

// The codes of e4m3_quant2_exact for a scale 0 < s < kTinyScale.
__device__ __forceinline__ uint32_t e4m3_quant2_tiny(float v0, float v1, float s) {
    const float sl = s * kTinyLift;
    return e4m3_quant2_exact(v0 * kTinyLift, v1 * kTinyLift, sl, 1.0f / sl);
}

// The same codes, always resolved, for any scale s > 0 (r = fp32(1 / s) is used when
// s >= kTinyScale).
__device__ __forceinline__ uint32_t e4m3_quant2(float v0, float v1, float s, float r) {
    return s < kTinyScale ? e4m3_quant2_tiny(v0, v1, s) : e4m3_quant2_exact(v0, v1, s, r);
}

__host__ __device__ __forceinline__ float bf16_to_float(uint16_t b) {
    return u2f((uint32_t)b << 16);
}

// float32 -> bf16, round to nearest even (finite inputs).
__host__ __device__ __forceinline__ uint16_t float_to_bf16(float f) {
    const uint32_t u = f2u(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

}  // namespace moe
