// Test-only host build of the device group quantiser (quantized_kv_decode_amd/csrc/quantize.h),
// so that its integer and floating-point decision logic can be checked against the oracle
// without a GPU. The device builtins are replaced by host code:
//   * v_perm_b32: byte select from the 8-byte concatenation S0:S1;
//   * the fp64 reciprocal, perturbed by a relative eps so that the candidate correction of
//     the exact scale decision is exercised;
//   * the fp32 reciprocal, perturbed by eps clamped to +-2^-22 (twice the hardware's
//     one-ulp bound; the fast path's bracket relies on that bound);
//   * the fp32 -> E2M1 (scale 1) and fp32 -> E4M3FN conversions: nearest code, ties to
//     the even code, sign kept, E2M1 saturating at 6, E4M3 NaN (0x7F) above 464 -- what
//     the hardware instructions do on every input that quantize.h gives them.
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

#define __device__
static inline uint32_t host_perm(uint32_t s0, uint32_t s1, uint32_t sel) {
    const uint64_t v = ((uint64_t)s0 << 32) | s1;
    uint32_t r = 0;
    for (int i = 0; i < 4; ++i) {
        const uint32_t s = (sel >> (8 * i)) & 0xFFu;   // only selectors 0..7 are used
        r |= (uint32_t)((v >> (8 * s)) & 0xFFu) << (8 * i);
    }
    return r;
}
static double rcp_eps = 0.0;
static inline double host_rcp(double x) { return (1.0 / x) * (1.0 + rcp_eps); }
static inline float host_rcpf(float x) {
    const double e = fmin(fmax(rcp_eps, -0x1p-22), 0x1p-22);
    return (float)((1.0 / (double)x) * (1.0 + e));
}
static inline int min(int a, int b) { return a < b ? a : b; }
static inline uint32_t max(uint32_t a, uint32_t b) { return a > b ? a : b; }

// E2M1 magnitude code of a >= 0: nearest of 0, 0.5, 1, 1.5, 2, 3, 4, 6, ties to the even code.
static uint32_t host_e2m1(double a) {
    static const double v[8] = {0, 0.5, 1, 1.5, 2, 3, 4, 6};
    for (int c = 0; c < 7; ++c) {
        if (a < v[c + 1]) {
            const double mid = 0.5 * (v[c] + v[c + 1]);
            return (uint32_t)(a < mid ? c : a > mid ? c + 1 : (c & 1) ? c + 1 : c);
        }
    }
    return 7;
}
static uint32_t host_fp4(float x) { return (signbit(x) ? 8u : 0u) | host_e2m1(fabs((double)x)); }
static uint32_t host_cvt_pk_fp4(uint32_t old, float a, float b, float scale, int sel) {
    if (scale != 1.0f) abort();
    const uint32_t byte = host_fp4(a) | (host_fp4(b) << 4);
    return (old & ~(0xFFu << (8 * sel))) | (byte << (8 * sel));
}
// E4M3FN code of x: nearest (ties to even) below 2^-6 on the subnormal grid 2^-9, else on the
// binade's grid of 8 steps (rint rounds to nearest even, and a code's parity is its step's).
static uint32_t host_fp8(float x) {
    const double a = fabs((double)x);
    const uint32_t sign = signbit(x) ? 0x80u : 0u;
    if (isnan(x) || a > 464.0) return sign | 0x7Fu;
    if (a < 0x1p-6) return sign | (uint32_t)rint(a * 512.0);
    int e;
    frexp(a, &e);                                  // a in [2^(e-1), 2^e)
    const double m = rint(ldexp(a, 4 - e));        // step 2^(e-4): m in [8, 16]
    const uint32_t c = (uint32_t)((e - 1 + 7) * 8 + (int)m - 8);
    return sign | (c > 0x7Eu ? 0x7Eu : c);
}
static int host_cvt_pk_fp8(float a, float b, int old, bool hi) {
    const uint32_t pair = host_fp8(a) | (host_fp8(b) << 8);
    return (int)(hi ? (((uint32_t)old & 0xFFFFu) | (pair << 16)) : (((uint32_t)old & 0xFFFF0000u) | pair));
}
#define __builtin_amdgcn_perm host_perm
#define __builtin_amdgcn_rcp host_rcp
#define __builtin_amdgcn_rcpf host_rcpf
#define __builtin_amdgcn_cvt_scalef32_pk_fp4_f32 host_cvt_pk_fp4
#define __builtin_amdgcn_cvt_pk_fp8_f32 host_cvt_pk_fp8
#include "quantize.h"

// x: n_groups x 16 bf16 bit patterns; g: one global scale per group. Writes 8 code bytes and
// one scale byte per group, in the pool's byte order.
extern "C" void quantize_groups(const uint16_t *x, long n_groups, const float *g, uint8_t *codes,
                                uint8_t *scales, double eps) {
    rcp_eps = eps;
    for (long i = 0; i < n_groups; ++i) {
        uint32_t w[8];
        for (int k = 0; k < 8; ++k) w[k] = x[16 * i + 2 * k] | ((uint32_t)x[16 * i + 2 * k + 1] << 16);
        uint32_t packed[2];
        scales[i] = (uint8_t)nvfp4::dev::quantize_group(w, g[i], packed);
        for (int k = 0; k < 8; ++k) codes[8 * i + k] = (uint8_t)(packed[k >> 2] >> (8 * (k & 3)));
    }
}

// Row-scaled FP8 E4M3 (K8V4's K rows): x n_rows x D bf16; codes n_rows x D; scales n_rows.
// The row maximum is reduced over the row's 16-element groups as the device reduces it
// across the lanes that hold them.
extern "C" void quantize_rows_fp8(const uint16_t *x, long n_rows, int D, uint8_t *codes, float *scales, double eps) {
    rcp_eps = eps;
    for (long r = 0; r < n_rows; ++r) {
        uint32_t amax = 0;
        for (int j = 0; j < D / 16; ++j) {
            uint32_t w[8];
            for (int k = 0; k < 8; ++k)
                w[k] = x[r * D + 16 * j + 2 * k] | ((uint32_t)x[r * D + 16 * j + 2 * k + 1] << 16);
            amax = max(amax, nvfp4::dev::amax16_bits(w));
        }
        const float s = nvfp4::dev::fp8_row_scale(amax);
        scales[r] = s;
        for (int j = 0; j < D / 16; ++j) {
            uint32_t w[8], out[4];
            for (int k = 0; k < 8; ++k)
                w[k] = x[r * D + 16 * j + 2 * k] | ((uint32_t)x[r * D + 16 * j + 2 * k + 1] << 16);
            nvfp4::dev::fp8_row_codes(w, s, out);
            for (int e = 0; e < 16; ++e) codes[r * D + 16 * j + e] = (uint8_t)(out[e >> 2] >> (8 * (e & 3)));
        }
    }
}
