// Test-only host build of the device group quantiser (quantized_kv_decode_amd/csrc/quantize.h),
// so that its integer and floating-point decision logic can be checked against the oracle
// without a GPU. Two device builtins are replaced by host code: v_perm_b32 (byte select
// from the 8-byte concatenation S0:S1) and the fp64 reciprocal, which is perturbed by a
// relative eps so that the candidate correction of the scale code is exercised.
#include <math.h>
#include <stdint.h>

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
static inline float host_rcpf(float x) { return (float)((1.0 / (double)x) * (1.0 + rcp_eps)); }
static inline int min(int a, int b) { return a < b ? a : b; }
static inline uint32_t max(uint32_t a, uint32_t b) { return a > b ? a : b; }
#define __builtin_amdgcn_perm host_perm
#define __builtin_amdgcn_rcp host_rcp
#define __builtin_amdgcn_rcpf host_rcpf
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
