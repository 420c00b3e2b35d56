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
// Everything is branch-free (one thread handles one group, so the cost is the
// instruction count). How the decisions are made exact:
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

// One group: w holds 16 bf16 values (element 2k in the low half of word k), g the
// global scale. Returns the E4M3 scale code; packed receives the 16 E2M1 codes,
// element 2j in the low nibble of byte j.
__device__ inline uint32_t quantize_group(const uint32_t (&w)[8], float g, uint32_t (&packed)[2]) {
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

// 16 elements of a row with row scale s -> 16 code bytes (element e in byte e of out).
// Rows with s >= 2^-60 (amax above 448 * 2^-60, every row that is not nearly zero) take the
// fp32 decision; smaller ones the fp64 one (both exact).
__device__ inline void fp8_row_codes(const uint32_t (&w)[8], float s, uint32_t (&out)[4]) {
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

}  // namespace dev
}  // namespace nvfp4
