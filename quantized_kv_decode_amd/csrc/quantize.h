// Quantise-on-append of one 16-element group, shared by the append kernel and the
// decode kernels that append the step's rows themselves (same code, same bits).
//
// Format (gzenz/ninfer page, "Context and model", NVFP4 KV cache bullet): 4-bit
// E2M1 codes, two per byte, with one E4M3 scale per 16 elements; here also a
// per-(sequence, KV head) fp32 global scale g = amax / 2688.
//
// Rounding is decided on exact reals. The group scale is the E4M3 value nearest
// amax/(6g) (ties to the even code, saturating at 448); each element's magnitude
// is the E2M1 value nearest |x|/(S g) (ties to the even code, saturating at 6).
// One thread handles one group, so the cost is the instruction count. Two ways to the
// same codes: the fast one (hardware conversions of bracketing fp32 quotients, with an
// exact fp32 test where the bounds round apart; at the end of this file) serves every
// group with a global (or row) scale in a normal range and finite inputs; the others take
// the exact decision below, which is branch-free. How the exact decision is made:
//   * scale: an approximate quotient gives the code c whose value is the largest
//     not above it; the exact code is c or c + 1 (the quotient is accurate to far
//     better than the 1/32 relative half-gap of E4M3), settled by one test against
//     the midpoint m(c, c+1), whose product with 6g is exact in fp64 (<= 32 bits);
//   * elements: the seven E2M1 midpoints t (0.25 ... 5) give thresholds T = t S g,
//     exact in fp64 (<= 31 bits). A bf16 input a compared with T is an fp32 value,
//     so "a > T" equals "a > rd32(T)" and "a >= T" equals "a > pred32(ru32(T))",
//     with rd32/ru32 the directed roundings to fp32. For non-negative floats the
//     order is the unsigned order of the bit patterns, and an fp32 threshold U
//     compares with a bf16 magnitude a16 as (a16 << 16) > U  <=>  a16 > (U >> 16).
//     So each group yields seven 16-bit integer thresholds, and every element is
//     classified by integer compares alone (exact, independent of denormal modes).
//     The compares run on two elements at once in 16-bit lanes: with u <= 0x7F80
//     and a16 <= 0x7FFF, the lane u - a16 is negative (bit 15 set) iff a16 > u.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace nvfp4 {
namespace dev {

typedef short s16x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ inline uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// E4M3FN code c (0..0x7E) has the value sig * 2^(ex - 10): exponent field 0 is
// subnormal (sig = mantissa, ex = 1), otherwise sig = 8 + mantissa, ex = field.
__device__ inline int e4m3_sig(int c) { return (c & 7) | (c >= 8 ? 8 : 0); }
__device__ inline int e4m3_ex(int c) { return c >= 8 ? (c >> 3) : 1; }

// Nearest E4M3 code to the real a / b, ties to even, saturating at 448; a >= 0, b > 0,
// rcp_b an approximation of 1 / b (relative error far below E4M3's 1/32 half-gap), and the
// product of b with a 5-bit midpoint exact in fp64 (b has at most 48 significant bits).
__device__ inline int e4m3_nearest(double a, double b, double rcp_b) {
    const double q = fmin(a * rcp_b, 448.0);
    const float q32 = (float)q;
    // Largest code whose value is at most q32 (values are monotone in the bits).
    const int c = q32 < 0.015625f ? (int)(q32 * 512.0f) : (int)(f32_bits(q32) >> 20) - 960;
    // m(c, c+1) * b = (2 sig + 1) 2^(ex - 11) * b, exact.
    const double mid = ldexp((double)(2 * e4m3_sig(c) + 1) * b, e4m3_ex(c) - 11);
    const int up = a > mid || (a == mid && (c & 1));         // tie: to the even one of c, c+1
    return min(c + up, 0x7E);
}

// Nearest E4M3 code to amax / (6 g), ties to even, saturating; amax > 0, g > 0 (6 g is exact).
__device__ inline int e4m3_code_exact(double amax, double gd) {
    return e4m3_nearest(amax, 6.0 * gd, __builtin_amdgcn_rcp(6.0 * gd));
}

// Both 16-bit lanes = the threshold for "a > T" (strict) or "a >= T".
__device__ inline uint32_t thr_pair(double T, bool strict) {
    const float f = (float)T;                         // to nearest
    const double back = (double)f;
    // strict: rd32(T) = f, or its predecessor when f rounded up;
    // else:   pred32(ru32(T)) = f's predecessor, or f when f rounded down.
    const uint32_t bits = f32_bits(f) - (uint32_t)(strict ? back > T : back >= T);
    return __builtin_amdgcn_perm(bits, bits, 0x03020302u);   // high half, twice
}

__device__ inline uint32_t pk_sub16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2_t, a) - __builtin_bit_cast(u16x2_t, b));
}
// 0xFFFF in each lane whose bit 15 is set. The empty asm hides that the result is a
// lane mask: knowing it, the compiler turns each bit select on it into two 16-bit
// selects and a repack (five instructions instead of one).
__device__ inline uint32_t pk_sign16(uint32_t a) {
    uint32_t m = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2_t, a) >> (short)15);
    asm("" : "+v"(m));
    return m;
}
__device__ inline uint32_t pk_max16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
}
__device__ inline uint32_t sel(uint32_t m, uint32_t x, uint32_t y) { return (m & x) | (~m & y); }

// Codes of the two elements of P (bf16 e in the low lane, e + 4 in the high lane),
// placed at nibble e of each 16-bit half: a three-level binary search over u[0..6].
template <int E>
__device__ inline uint32_t e2m1_pair(uint32_t P, const uint32_t (&u)[7]) {
    const uint32_t A = P & 0x7FFF7FFFu;
    const uint32_t m1 = pk_sign16(pk_sub16(u[3], A));
    const uint32_t m2 = pk_sign16(pk_sub16(sel(m1, u[5], u[1]), A));
    const uint32_t s3 = pk_sub16(sel(m1, sel(m2, u[6], u[4]), sel(m2, u[2], u[0])), A);
    constexpr uint32_t one = 0x00010001u << (4 * E);
    return (m1 & (one << 2)) | (m2 & (one << 1)) | ((s3 >> (15 - 4 * E)) & one) |
           ((P >> (12 - 4 * E)) & (one << 3));
}

// One group, exactly: w holds 16 bf16 values (element 2k in the low half of word k), g
// the global scale. Returns the E4M3 scale code; packed receives the 16 E2M1 codes,
// element 2j in the low nibble of byte j.
__device__ inline uint32_t quantize_group_exact(const uint32_t (&w)[8], float g, uint32_t (&packed)[2]) {
    // Pair element n (of each half of the group) with element n + 4, so that both
    // lanes of a pair land on the same nibble of their half of the packed word.
    uint32_t P[8];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        P[4 * h + 0] = __builtin_amdgcn_perm(w[4 * h + 2], w[4 * h + 0], 0x05040100u);
        P[4 * h + 1] = __builtin_amdgcn_perm(w[4 * h + 2], w[4 * h + 0], 0x07060302u);
        P[4 * h + 2] = __builtin_amdgcn_perm(w[4 * h + 3], w[4 * h + 1], 0x05040100u);
        P[4 * h + 3] = __builtin_amdgcn_perm(w[4 * h + 3], w[4 * h + 1], 0x07060302u);
    }
    uint32_t mx = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = pk_max16(mx, P[k] & 0x7FFF7FFFu);
    const uint32_t amax16 = max(mx & 0xFFFFu, mx >> 16);

    const double gd = (double)g;
    const double amax = (double)__builtin_bit_cast(float, amax16 << 16);
    const int sc = (g > 0.0f && amax16 != 0) ? e4m3_code_exact(amax, gd) : 0;
    // S g, exact (<= 28 significant bits); a zero scale maps every magnitude to 0,
    // which the infinite thresholds give.
    const double Sg = sc ? ldexp((double)e4m3_sig(sc) * gd, e4m3_ex(sc) - 10) : (double)INFINITY;

    uint32_t u[7];
    u[0] = thr_pair(0.25 * Sg, true);  u[1] = thr_pair(0.75 * Sg, false);
    u[2] = thr_pair(1.25 * Sg, true);  u[3] = thr_pair(1.75 * Sg, false);
    u[4] = thr_pair(2.5 * Sg, true);   u[5] = thr_pair(3.5 * Sg, false);
    u[6] = thr_pair(5.0 * Sg, true);
#pragma unroll
    for (int h = 0; h < 2; ++h)
        packed[h] = e2m1_pair<0>(P[4 * h + 0], u) | e2m1_pair<1>(P[4 * h + 1], u) |
                    e2m1_pair<2>(P[4 * h + 2], u) | e2m1_pair<3>(P[4 * h + 3], u);
    return (uint32_t)sc;
}

// ---- row-scaled FP8 E4M3 (the K rows of K8V4) ----------------------------------------
// A row of D bf16 values gets one fp32 scale s = fp32(amax_row / 448) (the fp64 quotient
// rounded to fp32 is the correctly rounded fp32 quotient) and element codes sign << 7 |
// the E4M3 value nearest the exact real |x| / s (e4m3_nearest: s has 24 significant bits,
// so every midpoint product is exact in fp64). s == 0 gives zero magnitudes.

// Largest bf16 magnitude bit pattern among 16 elements (w: element 2k in the low half of
// word k); magnitudes order like their bit patterns.
__device__ inline uint32_t amax16_bits(const uint32_t (&w)[8]) {
    uint32_t mx = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) mx = pk_max16(mx, w[k] & 0x7FFF7FFFu);
    return max(mx & 0xFFFFu, mx >> 16);
}

__device__ inline float fp8_row_scale(uint32_t amax_bits) {
    return (float)((double)__builtin_bit_cast(float, amax_bits << 16) / 448.0);
}

// Nearest E4M3 code to the real a / s in fp32 (a >= 0 a bf16 value, s >= 2^-60): the same
// candidate-and-one-midpoint-test decision as e4m3_nearest, with the test taken from the sign
// of fma(mid, s, -a). That sign is exact: fma rounds the exact mid s - a once, rounding (and
// overflow to infinity) keeps the sign, and a nonzero difference never rounds to zero. When a
// lies within a factor two of mid s >= 2^-70, both are multiples of 2^-93 (mid of 2^-10, s of
// 2^-83, a >= 2^-71 of 2^-78), far above fp32's smallest normal; otherwise the difference
// exceeds 2^-71 in size.
__device__ inline int e4m3_nearest_f32(float a, float s, float rcp_s) {
    const float q = fminf(a * rcp_s, 448.0f);
    const int c = q < 0.015625f ? (int)(q * 512.0f) : (int)(f32_bits(q) >> 20) - 960;
    const float mid = ldexpf((float)(2 * e4m3_sig(c) + 1), e4m3_ex(c) - 11);
    const float d = fmaf(mid, s, -a);
    const int up = d < 0.0f || (d == 0.0f && (c & 1));
    return min(c + up, 0x7E);
}

// 16 elements of a row with row scale s -> 16 code bytes (element e in byte e of out),
// exactly. Rows with s >= 2^-60 (amax above 448 * 2^-60, every row that is not nearly zero)
// take the fp32 decision; smaller ones the fp64 one (both exact).
__device__ inline void fp8_row_codes_exact(const uint32_t (&w)[8], float s, uint32_t (&out)[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) out[k] = 0u;
    if (s >= 0x1p-60f) {
        const float rs = __builtin_amdgcn_rcpf(s);
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
            const float a = __builtin_bit_cast(float, (h & 0x7FFFu) << 16);
            const int c = e4m3_nearest_f32(a, s, rs);
            out[e >> 2] |= ((uint32_t)c | ((h >> 8) & 0x80u)) << (8 * (e & 3));
        }
        return;
    }
    const double sd = (double)s;
    const double rs = __builtin_amdgcn_rcp(sd);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
        const uint32_t h = (w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        const double a = (double)__builtin_bit_cast(float, (h & 0x7FFFu) << 16);
        const int c = s > 0.0f ? e4m3_nearest(a, sd, rs) : 0;
        out[e >> 2] |= ((uint32_t)c | ((h >> 8) & 0x80u)) << (8 * (e & 3));
    }
}

// ---- the fast path: hardware round-to-nearest conversions of bracketing quotients --------
// gfx950's v_cvt_scalef32_pk_fp4_f32 (with scale 1) and v_cvt_pk_fp8_f32 round an fp32
// value to the nearest E2M1 / E4M3FN code, ties to the even code, sign kept; E2M1 saturates
// at 6, E4M3 gives NaN above 464, so a quotient that may exceed 448 is clamped to 448 first.
// Rounding to nearest is monotone. If lo <= x <= hi and the codes of lo and hi are equal,
// that code is x's own nearest code. The bounds of a quotient a / b are a * r (1 -+ 2^-19)
// in fp32, with r = v_rcp_f32 (within one ulp) of the fp32-rounded b: the reciprocal's error
// and the three roundings stay below 2^-22 relative, far inside the 2^-19 margin, while
// every operand is a normal number (group divisors within 2^-109..2^109, FP8 row scales
// within 2^-100..2^120, so every reciprocal is normal; a product that underflows lies far
// below the first midpoint, where both bounds give code 0).
//
// Where the two codes differ, a midpoint m lies between the bounds (one only: midpoints are
// far more than 2^-18 apart, so the codes are c and c + 1), and the exact code is c + [a >
// m b] (a tie to the even one). That test is exact in fp32: m b = p + e with p = fl(m b) and
// e = fma(m, b, -p) (m has at most seven significant bits, so the product's bits and its
// residual are representable, subnormal residuals included, for b >= 2^-109; m b stays
// finite, being within 2^-17 of a finite input), and a - p is exact because a lies within a
// factor (1 +- 2^-17) of m b (Sterbenz); so a - m b has the sign of (a - p) - e. Such quotients are common: with g = amax / 2688 and bf16 inputs
// (8-bit significands), many are a midpoint times (1 + the rounding error of g). Only scales
// outside the ranges above, or non-finite inputs, take the exact decision of the first part.
constexpr float kBelow = 0x1.ffffcp-1f;        // 1 - 2^-19
constexpr float kAbove = 0x1.00002p+0f;        // 1 + 2^-19

__device__ inline float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xFFFF0000u); }

// E2M1 codes of word K's two elements times r into byte K % 4 of c.
template <int K>
__device__ inline uint32_t fp4_pair(uint32_t c, uint32_t w, float r) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c, bf16_lo(w) * r, bf16_hi(w) * r, 1.0f, K & 3);
}
// E4M3 codes of word K's two elements times r into bytes 2 (K % 2), 2 (K % 2) + 1 of c.
template <int K>
__device__ inline uint32_t fp8_pair(uint32_t c, uint32_t w, float r) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(bf16_lo(w) * r, bf16_hi(w) * r, (int)c, (K & 1) != 0);
}

// E4M3 value of code c (0..0x7E) as fp32: subnormal c * 2^-9, else exponent and mantissa
// fields moved into place.
__device__ inline float e4m3_f32(uint32_t c) {
    return c < 8 ? (float)c * 0x1p-9f : __builtin_bit_cast(float, (c << 20) + (120u << 23));
}

// E2M1 midpoint between magnitude codes c and c + 1 (c = 0..6): 0.25, 0.75, 1.25, 1.75,
// 2.5, 3.5, 5.
__device__ inline float e2m1_mid(uint32_t c) {
    const float f = (float)c;
    return c < 4 ? 0.5f * f + 0.25f : (c == 6 ? 5.0f : f - 1.5f);
}

// 1 if the real a / b lies above m, or on it with c odd (a tie goes to the even one of c,
// c + 1); a, m, b > 0 under the conditions stated above.
__device__ inline uint32_t above_mid(float a, float m, float b, uint32_t c) {
#pragma clang fp contract(off)
    const float p = m * b;
    const float e = fmaf(m, b, -p);
    const float d = a - p;
    return (uint32_t)(d > e || (d == e && (c & 1u)));
}

// above_mid for an element whose bounds rounded apart around m: its magnitude a is a bf16
// value within a factor (1 +- 2^-17) of m b, and bf16 values lie at least 2^-8 apart
// (relative; subnormal ones further), so a is the bf16 value nearest fl(m b) -- the test
// needs neither the element nor its position.
__device__ inline uint32_t above_mid_bf16(float m, float b, uint32_t c) {
#pragma clang fp contract(off)
    const float p = m * b;
    const float e = fmaf(m, b, -p);
    const float a = __builtin_bit_cast(float, (__builtin_bit_cast(uint32_t, p) + 0x8000u) & 0xFFFF0000u);
    const float d = a - p;
    return (uint32_t)(d > e || (d == e && (c & 1u)));
}

// Codes lo (E2M1, nibbles) where they differ from hi, for group scale value S and global
// scale g (midpoint * S exact: at most seven significant bits).
__device__ inline uint32_t settle_e2m1(uint32_t lo, uint32_t hi, float S, float g) {
    uint32_t dm = lo ^ hi;
    while (dm) {
        const uint32_t sh = (uint32_t)__builtin_ctz(dm) & ~3u;
        const uint32_t c = (lo >> sh) & 7u;
        lo += above_mid_bf16(e2m1_mid(c) * S, g, c) << sh;
        dm &= ~(0xFu << sh);
    }
    return lo;
}

// Codes lo (E4M3, bytes) where they differ from hi, for row scale s.
__device__ inline uint32_t settle_e4m3(uint32_t lo, uint32_t hi, float s) {
    uint32_t dm = lo ^ hi;
    while (dm) {
        const uint32_t sh = (uint32_t)__builtin_ctz(dm) & ~7u;
        const uint32_t c = (lo >> sh) & 0x7Fu;
        const float m = (e4m3_f32(c) + e4m3_f32(c + 1)) * 0.5f;    // exact
        lo += above_mid_bf16(m, s, c) << sh;
        dm &= ~(0xFFu << sh);
    }
    return lo;
}

// One group: the same codes as quantize_group_exact. Returns the E4M3 scale code; packed
// receives the 16 E2M1 codes, element 2j in the low nibble of byte j.
__device__ inline uint32_t quantize_group(const uint32_t (&w)[8], float g, uint32_t (&packed)[2]) {
    const uint32_t amax16 = amax16_bits(w);
    if (!(g >= 0x1p-100f && g <= 0x1p100f && amax16 < 0x7F80u)) return quantize_group_exact(w, g, packed);
    const float amax = __builtin_bit_cast(float, amax16 << 16);
    const float r6 = __builtin_amdgcn_rcpf(6.0f * g);
    const uint32_t q2 = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(amax * (r6 * kBelow), 448.0f),
                                                                  fminf(amax * (r6 * kAbove), 448.0f), 0, false);
    uint32_t sc = q2 & 0xFFu;
    if (sc != ((q2 >> 8) & 0xFFu))                    // 6 * the midpoint above sc, exact
        sc += above_mid(amax, (e4m3_f32(sc) + e4m3_f32(sc + 1)) * 3.0f, g, sc);
    const float S = e4m3_f32(sc);
    const float r = sc ? __builtin_amdgcn_rcpf(S * g) : 0.0f;
    const float rl = r * kBelow, rh = r * kAbove;
    uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};
    lo[0] = fp4_pair<0>(lo[0], w[0], rl); hi[0] = fp4_pair<0>(hi[0], w[0], rh);
    lo[0] = fp4_pair<1>(lo[0], w[1], rl); hi[0] = fp4_pair<1>(hi[0], w[1], rh);
    lo[0] = fp4_pair<2>(lo[0], w[2], rl); hi[0] = fp4_pair<2>(hi[0], w[2], rh);
    lo[0] = fp4_pair<3>(lo[0], w[3], rl); hi[0] = fp4_pair<3>(hi[0], w[3], rh);
    lo[1] = fp4_pair<4>(lo[1], w[4], rl); hi[1] = fp4_pair<4>(hi[1], w[4], rh);
    lo[1] = fp4_pair<5>(lo[1], w[5], rl); hi[1] = fp4_pair<5>(hi[1], w[5], rh);
    lo[1] = fp4_pair<6>(lo[1], w[6], rl); hi[1] = fp4_pair<6>(hi[1], w[6], rh);
    lo[1] = fp4_pair<7>(lo[1], w[7], rl); hi[1] = fp4_pair<7>(hi[1], w[7], rh);
    packed[0] = settle_e2m1(lo[0], hi[0], S, g);
    packed[1] = settle_e2m1(lo[1], hi[1], S, g);
    return sc;
}

// 16 elements of a row with row scale s = fp32(amax_row / 448): the same codes as
// fp8_row_codes_exact (element e in byte e of out). Quotients stay below
// 448 (1 + 2^-18) < 464, so no clamp is needed.
__device__ inline void fp8_row_codes(const uint32_t (&w)[8], float s, uint32_t (&out)[4]) {
    if (!(s >= 0x1p-100f && s <= 0x1p120f)) {
        fp8_row_codes_exact(w, s, out);
        return;
    }
    const float r = __builtin_amdgcn_rcpf(s);
    const float rl = r * kBelow, rh = r * kAbove;
    uint32_t lo[4] = {0u, 0u, 0u, 0u}, hi[4] = {0u, 0u, 0u, 0u};
    lo[0] = fp8_pair<0>(lo[0], w[0], rl); hi[0] = fp8_pair<0>(hi[0], w[0], rh);
    lo[0] = fp8_pair<1>(lo[0], w[1], rl); hi[0] = fp8_pair<1>(hi[0], w[1], rh);
    lo[1] = fp8_pair<2>(lo[1], w[2], rl); hi[1] = fp8_pair<2>(hi[1], w[2], rh);
    lo[1] = fp8_pair<3>(lo[1], w[3], rl); hi[1] = fp8_pair<3>(hi[1], w[3], rh);
    lo[2] = fp8_pair<4>(lo[2], w[4], rl); hi[2] = fp8_pair<4>(hi[2], w[4], rh);
    lo[2] = fp8_pair<5>(lo[2], w[5], rl); hi[2] = fp8_pair<5>(hi[2], w[5], rh);
    lo[3] = fp8_pair<6>(lo[3], w[6], rl); hi[3] = fp8_pair<6>(hi[3], w[6], rh);
    lo[3] = fp8_pair<7>(lo[3], w[7], rl); hi[3] = fp8_pair<7>(hi[3], w[7], rh);
#pragma unroll
    for (uint32_t k = 0; k < 4; ++k) out[k] = settle_e4m3(lo[k], hi[k], s);
}

}  // namespace dev
}  // namespace nvfp4
