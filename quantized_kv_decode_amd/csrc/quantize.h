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
// How the decisions are made exact:
//   * scale: a candidate from the fp64 quotient, then one correction against the
//     neighbouring midpoints m with exact fp64 products m * 6g (<= 31 bits);
//   * elements: the seven E2M1 midpoints t (0.25 ... 5) give thresholds T = t S g,
//     exact in fp64 (<= 31 bits). A bf16 input a compared with T is an fp32 value,
//     so "a > T" equals "a > rd32(T)" and "a >= T" equals "a > pred32(ru32(T))",
//     with rd32/ru32 the directed roundings to fp32. For non-negative floats the
//     order is the unsigned order of the bit patterns, and an fp32 threshold U
//     compares with a bf16 magnitude a16 as (a16 << 16) > U  <=>  a16 > (U >> 16).
//     So each group yields seven 16-bit integer thresholds and every element is
//     classified by integer compares alone (exact, independent of denormal modes).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

namespace nvfp4 {
namespace dev {

// E4M3FN value of a non-negative code 0x00..0x7E: exponent field 0 is subnormal.
__device__ inline double e4m3_pos_value(int c) {
    const int e = c >> 3, m = c & 7;
    return e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
}

// Nearest E4M3 code to amax / b6 (b6 = 6 g > 0, exact), ties to even, saturating.
__device__ inline int e4m3_code_exact(double amax, double b6) {
    const double q = amax / b6;                       // correctly rounded fp64
    int c;
    if (!(q < 448.0)) {
        c = 0x7E;
    } else if (q < 0.015625) {                        // below 2^-6: subnormal spacing 2^-9
        c = (int)rint(q * 512.0);                     // 0..8 (8 = 2^-6, the first normal)
    } else {
        int e;
        const double f = frexp(q, &e);                // q = f * 2^e, f in [0.5, 1)
        const int m = (int)rint(f * 16.0) - 8;        // 3-bit mantissa, may carry to 8
        c = ((e + 6) << 3) + m;                       // exponent field e - 1 + 7
        if (c > 0x7E) c = 0x7E;
    }
    // The fp64 quotient differs from the exact one by < 1 ulp, so the candidate is
    // at most one code away; settle with the exact midpoint tests.
    if (c < 0x7E) {
        const double up = 0.5 * (e4m3_pos_value(c) + e4m3_pos_value(c + 1)) * b6;
        if (amax > up || (amax == up && ((c + 1) & 1) == 0)) return c + 1;
    }
    if (c > 0) {
        const double dn = 0.5 * (e4m3_pos_value(c - 1) + e4m3_pos_value(c)) * b6;
        if (amax < dn || (amax == dn && ((c - 1) & 1) == 0)) return c - 1;
    }
    return c;
}

__device__ inline uint32_t f32_bits(float f) { return __builtin_bit_cast(uint32_t, f); }

// Round a positive double to fp32 downward / upward.
__device__ inline float rd32(double t) {
    float f = (float)t;
    if ((double)f > t) f = nextafterf(f, 0.0f);
    return f;
}
__device__ inline float ru32(double t) {
    float f = (float)t;
    if ((double)f < t) f = nextafterf(f, INFINITY);
    return f;
}

// 16-bit threshold for "a > t*Sg" (strict: ties go down) and "a >= t*Sg" (ties go up).
__device__ inline uint32_t thr_gt(double T) { return f32_bits(rd32(T)) >> 16; }
__device__ inline uint32_t thr_ge(double T) {
    const float u = ru32(T);
    return f32_bits(nextafterf(u, 0.0f)) >> 16;     // u > 0 here
}

// The group's seven thresholds, u_k <-> midpoint k in (0.25 >, 0.75 >=, 1.25 >, 1.75 >=,
// 2.5 >, 3.5 >=, 5 >).
struct Thresholds {
    uint32_t u0, u1, u2, u3, u4, u5, u6;
};

// Magnitude code of a bf16 magnitude a16: a three-level binary search over the thresholds.
// The thresholds come by value: selecting between members of a referenced struct is
// turned into a computed-offset load, which keeps the struct in private memory.
__device__ inline uint32_t e2m1_mag(uint32_t a16, const Thresholds t) {
    const uint32_t c1 = a16 > t.u3;
    const uint32_t c2 = a16 > (c1 ? t.u5 : t.u1);
    const uint32_t t3 = c1 ? (c2 ? t.u6 : t.u4) : (c2 ? t.u2 : t.u0);
    const uint32_t c3 = a16 > t3;
    return (c1 << 2) | (c2 << 1) | c3;
}

// One group: w holds 16 bf16 values (element 2k in the low half of word k), g the
// global scale. Returns the E4M3 scale code; packed receives the 16 E2M1 codes,
// element 2j in the low nibble of byte j.
__device__ inline uint32_t quantize_group(const uint32_t (&w)[8], double g, uint32_t (&packed)[2]) {
    uint32_t amax16 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        amax16 = max(amax16, w[k] & 0x7FFFu);
        amax16 = max(amax16, (w[k] >> 16) & 0x7FFFu);
    }
    const double amax = (double)__builtin_bit_cast(float, amax16 << 16);
    int sc = 0;
    if (g > 0.0 && amax > 0.0) sc = e4m3_code_exact(amax, 6.0 * g);
    const double Sg = e4m3_pos_value(sc) * g;        // exact (<= 28 significant bits)

    Thresholds u;
    if (Sg > 0.0) {
        u.u0 = thr_gt(0.25 * Sg); u.u1 = thr_ge(0.75 * Sg); u.u2 = thr_gt(1.25 * Sg);
        u.u3 = thr_ge(1.75 * Sg); u.u4 = thr_gt(2.5 * Sg);  u.u5 = thr_ge(3.5 * Sg);
        u.u6 = thr_gt(5.0 * Sg);
    } else {
        u.u0 = u.u1 = u.u2 = u.u3 = u.u4 = u.u5 = u.u6 = 0xFFFFu;   // every magnitude 0
    }
    packed[0] = packed[1] = 0u;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t lo = w[k] & 0xFFFFu, hi = w[k] >> 16;
        const uint32_t c0 = e2m1_mag(lo & 0x7FFFu, u) | ((lo >> 12) & 8u);
        const uint32_t c1 = e2m1_mag(hi & 0x7FFFu, u) | ((hi >> 12) & 8u);
        packed[k >> 2] |= (c0 | (c1 << 4)) << (8 * (k & 3));
    }
    return (uint32_t)sc;
}

}  // namespace dev
}  // namespace nvfp4
