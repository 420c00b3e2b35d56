/* Sanitizer driver for the CPU oracle (oracle/nvfp4_oracle.c), built with gcc
 * -fsanitize=address,undefined by tests/test_sanitizers.py: quantises NVFP4 and row-scaled
 * FP8 rows (random values over many decades, zeros, signed zeros, bf16 subnormals and the
 * largest bf16), dequantises them, and runs attention over both K formats with ragged
 * sequences on several threads. Any out-of-bounds access, leak or undefined behaviour aborts
 * the run; the driver itself only checks that results are finite. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void orc_quantize_rows(const uint16_t *, int64_t, int32_t, const float *, uint8_t *, uint8_t *, int);
void orc_dequantize_rows(const uint8_t *, const uint8_t *, int64_t, int32_t, const float *, double *);
void orc_quantize_rows_fp8(const uint16_t *, int64_t, int32_t, uint8_t *, float *, int);
void orc_dequantize_rows_fp8(const uint8_t *, const float *, int64_t, int32_t, double *);
float orc_global_scale(const uint16_t *, int64_t);
int orc_attention(const uint8_t *, const uint8_t *, const uint8_t *, const uint8_t *, int32_t, int32_t, int32_t,
                  int64_t, const float *, const uint16_t *, int32_t, const int64_t *, const int64_t *, int32_t,
                  int32_t, double, int64_t, const int32_t *, double *, int);

static uint32_t rng = 12345u;
static uint32_t next(void) { rng = rng * 1664525u + 1013904223u; return rng; }
static uint16_t rand_bf16(void) {
    uint32_t r = next();
    switch (r % 16) {
        case 0: return 0;
        case 1: return 0x8000;
        case 2: return (uint16_t)(1 + (r >> 8) % 0x7F);              /* bf16 subnormal */
        case 3: return 0x7F7F;                                      /* largest finite */
        default: {
            uint16_t e = (uint16_t)(100 + (r >> 4) % 60);           /* exponents 2^-27 .. 2^32 */
            return (uint16_t)(((r >> 16) & 0x8000) | (e << 7) | ((r >> 20) & 0x7F));
        }
    }
}

int main(void) {
    const int D = 256, H = 2, B = 3, nq = 3, Hq = 6;
    const int64_t lens[3] = {41, 3, 70}, base[3] = {0, 41, 44};
    const int64_t cap = 114;
    uint16_t *x = malloc(sizeof(uint16_t) * H * cap * D);
    for (int64_t i = 0; i < H * cap * D; ++i) x[i] = rand_bf16();
    /* planes [H][cap][...], rows of head h contiguous */
    uint8_t *kc4 = malloc(H * cap * D / 2), *ks4 = malloc(H * cap * D / 16);
    uint8_t *vc = malloc(H * cap * D / 2), *vs = malloc(H * cap * D / 16);
    uint8_t *kc8 = malloc(H * cap * D);
    float *ks8 = malloc(sizeof(float) * H * cap);
    float g[3 * 2 * 2];
    float *grow = malloc(sizeof(float) * H * cap);
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < H; ++h) {
            g[(b * H + h) * 2 + 0] = orc_global_scale(x + (h * cap + base[b]) * D, lens[b] * D);
            g[(b * H + h) * 2 + 1] = g[(b * H + h) * 2 + 0] * 0.5f;
            for (int64_t t = 0; t < lens[b]; ++t) grow[h * cap + base[b] + t] = g[(b * H + h) * 2 + 0];
        }
    orc_quantize_rows(x, H * cap, D, grow, kc4, ks4, 4);
    orc_quantize_rows(x, H * cap, D, grow, vc, vs, 3);
    orc_quantize_rows_fp8(x, H * cap, D, kc8, ks8, 4);
    double *dq = malloc(sizeof(double) * H * cap * D);
    orc_dequantize_rows(vc, vs, H * cap, D, grow, dq);
    orc_dequantize_rows_fp8(kc8, ks8, H * cap, D, dq);
    uint16_t *q = malloc(sizeof(uint16_t) * B * nq * Hq * D);
    for (int64_t i = 0; i < (int64_t)B * nq * Hq * D; ++i) q[i] = (uint16_t)(0x3C00 + next() % 0x200) ^ (next() & 0x8000);
    int32_t *sel = malloc(sizeof(int32_t) * 3 * B * nq * Hq);
    int n = 0;
    for (int b = 0; b < B; ++b)
        for (int i = 0; i < nq; ++i)
            for (int h = 0; h < Hq; ++h) { sel[3 * n] = b; sel[3 * n + 1] = i; sel[3 * n + 2] = h; ++n; }
    double *out = malloc(sizeof(double) * n * D);
    int bad = 0;
    for (int fmt = 0; fmt < 2; ++fmt) {
        int rc = orc_attention(fmt ? kc8 : kc4, fmt ? (const uint8_t *)ks8 : ks4, vc, vs, fmt, H, D, cap, g, q, B,
                               base, lens, nq, Hq, 0.0625, n, sel, out, 5);
        if (rc != 0) { printf("attention rc %d\n", rc); return 1; }
        for (int64_t i = 0; i < (int64_t)n * D; ++i) bad += !isfinite(out[i]);
    }
    /* invalid arguments are rejected, not read */
    sel[0] = 7;
    if (orc_attention(kc4, ks4, vc, vs, 0, H, D, cap, g, q, B, base, lens, nq, Hq, 0.0625, n, sel, out, 2) != -1) return 1;
    free(x); free(kc4); free(ks4); free(vc); free(vs); free(kc8); free(ks8); free(grow); free(dq); free(q);
    free(sel); free(out);
    printf("oracle sanitizer run: %d non-finite outputs\n", bad);
    return bad ? 1 : 0;
}
