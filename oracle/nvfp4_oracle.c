/*
 * NVFP4-KV CPU oracle: a plain, slow, fp64 implementation of what the GPU path
 * computes. TEST INFRASTRUCTURE ONLY: tests, the smoke check and the benchmark's
 * CPU-baseline leg load this library; the product path never does. It shares no
 * code, header, table or constant with the HIP kernels.
 *
 * What the method is, as the pages state it (gzenz/ninfer page, section "Context
 * and model", bullet "NVFP4 KV cache"): K and V are stored as 4-bit E2M1 codes
 * with one E4M3 scale per group of 16 elements. The pages say nothing more; every
 * other rule below is a stated reading (the design document lists them):
 *   - a second-level fp32 scale g per (sequence, KV head), one for K and one for
 *     V, g = fp32(amax / (6 * 448)) over that head's rows;
 *   - E2M1 and E4M3 are the OCP Microscaling v1.0 element formats (E4M3 = "FN":
 *     bias 7, max 448, 0x7F/0xFF NaN, no infinities);
 *   - the group scale S is the E4M3 value nearest the exact real amax_group/(6g),
 *     ties to the even code, saturating at 448; the element code is the E2M1 value
 *     nearest the exact real |x|/(S g), ties to the even code, saturating at 6, with
 *     the input's sign bit copied into the code's sign bit;
 *   - codes are packed two per byte, even element in the low nibble; scale byte j
 *     covers elements [16j, 16j + 16) of the row;
 *   - decode attention is plain softmax attention over the dequantised rows
 *     x_hat = e2m1(code) * S * g, with query head h reading KV head h / (Hq/Hkv) and
 *     query token i of n_q seeing keys [0, L - n_q + i] (the n_q query tokens' own
 *     K/V are the last n_q rows of the context).
 *
 * K8V4 (knoopx/ninfer page, "Capabilities and limits", KV storage list: 8-bit K with 4-bit
 * V) is stored with K as row-scaled FP8 E4M3 (the 8-bit K format is not given there; this
 * reading takes the engine's row-scaled FP8 E4M3 storage, knoopx/ninfer page, "Performance":
 * "FP8 E4M3 row-256", one scale per 256-element row, and gzenz/ninfer page, "Capabilities and
 * limits"): per (token, KV head) row, s = fp32(amax_row / 448) and each element's code is the
 * E4M3 value nearest the exact real x / s (ties to the even code, saturating at 448, sign bit
 * copied); x_hat = e4m3(code) * s. V is NVFP4 as above.
 *
 * Exactness of the rounding decisions. Every comparison below is of the form
 * a (vs) t * b with a exact and t * b an exact fp64 product:
 *   - scale:   a = amax (a bf16 value), b = 6 g (g has 24 significant bits, so 6 g
 *              has at most 26), t = an E4M3 midpoint (at most 5 significant bits):
 *              t * b has at most 31 significant bits < 53;
 *   - element: a = |x| (bf16), b = S g (S at most 4 significant bits: 28 in all),
 *              t = an E2M1 midpoint in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}
 *              (at most 3 bits): at most 31 significant bits.
 * No product can overflow or underflow fp64 for finite fp32 g. The decisions are
 * therefore the exact-real ones, independent of any rounding in this code.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------- formats */

/* E2M1 (OCP MX v1.0): bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent 0 is subnormal: 0.5 * m. */
double orc_e2m1_value(int code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN (OCP MX v1.0): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa. Exponent 0 is subnormal: m * 2^-9. S.1111.111 is NaN; no infinity. */
double orc_e4m3_value(int byte)
{
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

static double E2M1_MAG[8];    /* magnitudes of codes 0..7, increasing */
static double E4M3_POS[127];  /* values of codes 0x00..0x7E, increasing */
static double E2M1_ALL[16];   /* value of every code, filled from orc_e2m1_value */
static double E4M3_ALL[256];  /* value of every byte, filled from orc_e4m3_value */
static pthread_once_t tables_once = PTHREAD_ONCE_INIT;

static void build_tables(void)
{
    for (int c = 0; c < 8; ++c) E2M1_MAG[c] = orc_e2m1_value(c);
    for (int c = 0; c < 127; ++c) E4M3_POS[c] = orc_e4m3_value(c);
    for (int c = 0; c < 16; ++c) E2M1_ALL[c] = orc_e2m1_value(c);
    for (int c = 0; c < 256; ++c) E4M3_ALL[c] = orc_e4m3_value(c);
}

static void tables(void) { pthread_once(&tables_once, build_tables); }

/* Index of the entry of the increasing list vals[0..n) nearest the real a/b
 * (a >= 0, b > 0), ties to the even index, saturating at n - 1. The entry j+1 is
 * preferred over entry j exactly when a/b lies above their midpoint, i.e. when
 * a > mid * b (or a == mid * b and j + 1 is even). */
static int nearest_even(double a, double b, const double *vals, int n)
{
    int k = 0;
    for (int j = 0; j + 1 < n; ++j) {
        double mid_b = 0.5 * (vals[j] + vals[j + 1]) * b;
        if (a > mid_b) {
            k = j + 1;
        } else {
            if (a == mid_b) k = (j % 2 == 0) ? j : j + 1;
            break;
        }
    }
    return k;
}

/* E4M3 code (0x00..0x7E) nearest a/b; b <= 0 gives code 0. */
int orc_e4m3_encode(double a, double b)
{
    tables();
    if (!(b > 0.0)) return 0;
    return nearest_even(a, b, E4M3_POS, 127);
}

/* E2M1 magnitude code (0..7) nearest a/b; b <= 0 gives code 0. */
int orc_e2m1_encode(double a, double b)
{
    tables();
    if (!(b > 0.0)) return 0;
    return nearest_even(a, b, E2M1_MAG, 8);
}

static double bf16_value(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* g = fp32(amax / 2688) over n bf16 values. The fp64 quotient rounded once more
 * to fp32 equals the correctly rounded fp32 quotient (53 >= 2 * 24 + 2). */
float orc_global_scale(const uint16_t *x, int64_t n)
{
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) {
        double v = fabs(bf16_value(x[i]));
        if (v > amax) amax = v;
    }
    return (float)(amax / 2688.0);
}

/* Quantise one row of D bf16 values with global scale g into D/2 code bytes and
 * D/16 E4M3 scale bytes. */
static void quantize_row(const uint16_t *x, int32_t D, float g, uint8_t *codes, uint8_t *scales)
{
    double gd = (double)g;
    for (int32_t j = 0; j < D / 16; ++j) {
        const uint16_t *grp = x + 16 * j;
        double amax = 0.0;
        for (int i = 0; i < 16; ++i) {
            double v = fabs(bf16_value(grp[i]));
            if (v > amax) amax = v;
        }
        int sc = orc_e4m3_encode(amax, 6.0 * gd);
        double Sg = E4M3_POS[sc] * gd;
        scales[j] = (uint8_t)sc;
        for (int i = 0; i < 16; ++i) {
            int sign = (grp[i] >> 15) & 1;
            int mag = orc_e2m1_encode(fabs(bf16_value(grp[i])), Sg);
            int code = (sign << 3) | mag;
            int e = 16 * j + i;
            if (e % 2 == 0) codes[e / 2] = (uint8_t)code;
            else codes[e / 2] |= (uint8_t)(code << 4);
        }
    }
}

/* Row-scaled FP8 E4M3 (the K half of K8V4): s = fp32(amax / 448) over the row's D bf16
 * values (the fp64 quotient rounded once to fp32 is the correctly rounded fp32 quotient);
 * code d = sign(x_d) << 7 | the E4M3 magnitude code nearest |x_d| / s (exact: a midpoint
 * times s has at most 5 + 24 significant bits). s = 0 gives magnitude 0. */
static void quantize_row_fp8(const uint16_t *x, int32_t D, uint8_t *codes, float *scale)
{
    double amax = 0.0;
    for (int32_t d = 0; d < D; ++d) {
        double v = fabs(bf16_value(x[d]));
        if (v > amax) amax = v;
    }
    float s = (float)(amax / 448.0);
    *scale = s;
    for (int32_t d = 0; d < D; ++d) {
        int sign = (x[d] >> 15) & 1;
        int mag = orc_e4m3_encode(fabs(bf16_value(x[d])), (double)s);
        codes[d] = (uint8_t)((sign << 7) | mag);
    }
}

/* ----------------------------------------------------------- thread helper */

typedef void (*work_fn)(void *ctx, int64_t item);
typedef struct { work_fn fn; void *ctx; int64_t n; int tid, nthreads; } worker_arg;

static void *worker(void *p)
{
    worker_arg *a = (worker_arg *)p;
    for (int64_t i = a->tid; i < a->n; i += a->nthreads) a->fn(a->ctx, i);
    return NULL;
}

/* Runs fn(ctx, i) for i in [0, n) on nthreads threads (items are independent). */
static void parallel_for(work_fn fn, void *ctx, int64_t n, int nthreads)
{
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads == 1 || n < 2) {
        for (int64_t i = 0; i < n; ++i) fn(ctx, i);
        return;
    }
    pthread_t th[256];
    worker_arg args[256];
    for (int t = 0; t < nthreads; ++t) {
        args[t] = (worker_arg){fn, ctx, n, t, nthreads};
        pthread_create(&th[t], NULL, worker, &args[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------- quantise */

typedef struct {
    const uint16_t *x; int32_t D; const float *g; uint8_t *codes, *scales;
} quant_ctx;

static void quant_item(void *p, int64_t r)
{
    quant_ctx *c = (quant_ctx *)p;
    quantize_row(c->x + r * c->D, c->D, c->g[r], c->codes + r * (c->D / 2), c->scales + r * (c->D / 16));
}

/* Quantise n_rows rows of D bf16 values; g[r] is row r's global scale. */
void orc_quantize_rows(const uint16_t *x, int64_t n_rows, int32_t D, const float *g,
                       uint8_t *codes, uint8_t *scales, int nthreads)
{
    tables();
    quant_ctx c = {x, D, g, codes, scales};
    parallel_for(quant_item, &c, n_rows, nthreads);
}

typedef struct {
    const uint16_t *x; int32_t D; uint8_t *codes; float *scales;
} quant8_ctx;

static void quant8_item(void *p, int64_t r)
{
    quant8_ctx *c = (quant8_ctx *)p;
    quantize_row_fp8(c->x + r * c->D, c->D, c->codes + r * c->D, c->scales + r);
}

/* Row-scaled FP8 E4M3: n_rows rows of D bf16 values -> D code bytes and one fp32 scale each. */
void orc_quantize_rows_fp8(const uint16_t *x, int64_t n_rows, int32_t D, uint8_t *codes, float *scales,
                           int nthreads)
{
    tables();
    quant8_ctx c = {x, D, codes, scales};
    parallel_for(quant8_item, &c, n_rows, nthreads);
}

/* x_hat = e4m3(code) * s, one row of D values per r. */
void orc_dequantize_rows_fp8(const uint8_t *codes, const float *scales, int64_t n_rows, int32_t D, double *out)
{
    for (int64_t r = 0; r < n_rows; ++r)
        for (int32_t d = 0; d < D; ++d)
            out[r * D + d] = orc_e4m3_value(codes[r * D + d]) * (double)scales[r];
}

/* x_hat = e2m1(code) * e4m3(scale) * g, one row of D values per r. */
void orc_dequantize_rows(const uint8_t *codes, const uint8_t *scales, int64_t n_rows, int32_t D,
                         const float *g, double *out)
{
    for (int64_t r = 0; r < n_rows; ++r) {
        for (int32_t d = 0; d < D; ++d) {
            uint8_t byte = codes[r * (D / 2) + d / 2];
            int code = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
            out[r * D + d] = orc_e2m1_value(code) * orc_e4m3_value(scales[r * (D / 16) + d / 16]) * (double)g[r];
        }
    }
}

/* ------------------------------------------------------------ attention */

typedef struct {
    const uint8_t *kc, *ks, *vc, *vs;
    int32_t k_fp8;                 /* 0: K is NVFP4; 1: K is row-scaled FP8 E4M3 (K8V4) */
    int32_t Hkv, D; int64_t cap;
    const float *gscale;
    const uint16_t *q;
    const int64_t *seq_base, *seq_len;
    int32_t n_q, Hq; double sm_scale;
    const int32_t *sel; double *out;
    int status;
} attn_ctx;

/* Dequantised element d of token slot t of a head plane. */
static double khat(const uint8_t *codes, const uint8_t *scales, int32_t D, int64_t slot, int32_t d, double g)
{
    uint8_t byte = codes[slot * (D / 2) + d / 2];
    int code = (d % 2 == 0) ? (byte & 15) : (byte >> 4);
    return E2M1_ALL[code] * E4M3_ALL[scales[slot * (D / 16) + d / 16]] * g;
}

/* Element d of token slot t of a row-scaled FP8 head plane (codes [cap][D], scales [cap]). */
static double khat_fp8(const uint8_t *codes, const float *scales, int32_t D, int64_t slot, int32_t d)
{
    return E4M3_ALL[codes[slot * D + d]] * (double)scales[slot];
}

static void attn_item(void *p, int64_t n)
{
    attn_ctx *c = (attn_ctx *)p;
    int32_t b = c->sel[3 * n], i = c->sel[3 * n + 1], h = c->sel[3 * n + 2];
    int32_t D = c->D, G = c->Hq / c->Hkv, kh = h / G;
    int64_t L = c->seq_len[b], base = c->seq_base[b];
    int64_t nvis = L - c->n_q + i + 1;             /* keys 0 .. L - n_q + i */
    double gk = c->gscale[(b * c->Hkv + kh) * 2 + 0];
    double gv = c->gscale[(b * c->Hkv + kh) * 2 + 1];
    const uint16_t *qrow = c->q + (((int64_t)b * c->n_q + i) * c->Hq + h) * D;
    const uint8_t *kc = c->k_fp8 ? c->kc + (int64_t)kh * c->cap * D : c->kc + (int64_t)kh * c->cap * (D / 2);
    const uint8_t *ks = c->k_fp8 ? c->ks + (int64_t)kh * c->cap * 4 : c->ks + (int64_t)kh * c->cap * (D / 16);
    const uint8_t *vc = c->vc + (int64_t)kh * c->cap * (D / 2), *vs = c->vs + (int64_t)kh * c->cap * (D / 16);
    double *o = c->out + n * D;
    double *qd = (double *)malloc(sizeof(double) * D);
    double *s = (double *)malloc(sizeof(double) * (nvis > 0 ? nvis : 1));
    if (!qd || !s) { c->status = -1; free(qd); free(s); return; }
    for (int32_t d = 0; d < D; ++d) qd[d] = bf16_value(qrow[d]);

    /* scores s_p = sm_scale * sum_d q_d * k_hat[p, d] */
    double m = -INFINITY;
    for (int64_t t = 0; t < nvis; ++t) {
        double acc = 0.0;
        if (c->k_fp8)
            for (int32_t d = 0; d < D; ++d) acc += qd[d] * khat_fp8(kc, (const float *)ks, D, base + t, d);
        else
            for (int32_t d = 0; d < D; ++d) acc += qd[d] * khat(kc, ks, D, base + t, d, gk);
        s[t] = c->sm_scale * acc;
        if (s[t] > m) m = s[t];
    }
    /* softmax with the maximum subtracted, then the weighted sum of V rows */
    double z = 0.0;
    for (int64_t t = 0; t < nvis; ++t) { s[t] = exp(s[t] - m); z += s[t]; }
    for (int32_t d = 0; d < D; ++d) o[d] = 0.0;
    for (int64_t t = 0; t < nvis; ++t)
        for (int32_t d = 0; d < D; ++d) o[d] += s[t] * khat(vc, vs, D, base + t, d, gv);
    for (int32_t d = 0; d < D; ++d) o[d] /= z;
    free(qd);
    free(s);
}

/* Decode attention for the selected (b, i, h) triples sel[3n..3n+2]; out[n][D].
 * V planes are [Hkv][capacity][D/2] codes and [Hkv][capacity][D/16] scales; so are the K
 * planes when k_fp8 = 0, while k_fp8 = 1 (K8V4) takes K codes [Hkv][capacity][D] (E4M3) and
 * fp32 row scales [Hkv][capacity];
 * gscale is [B][Hkv][2] (0 = K, 1 = V); q is bf16 [B][n_q][Hq][D].
 * Returns 0, or -1 on bad arguments / allocation failure. */
int orc_attention(const uint8_t *k_codes, const uint8_t *k_scales, const uint8_t *v_codes,
                  const uint8_t *v_scales, int32_t k_fp8, int32_t Hkv, int32_t D, int64_t capacity,
                  const float *gscale, const uint16_t *q, int32_t B, const int64_t *seq_base,
                  const int64_t *seq_len, int32_t n_q, int32_t Hq, double sm_scale, int64_t n_sel,
                  const int32_t *sel, double *out, int nthreads)
{
    tables();
    if (Hkv <= 0 || D % 16 != 0 || Hq % Hkv != 0 || n_q <= 0) return -1;
    for (int64_t n = 0; n < n_sel; ++n) {
        int32_t b = sel[3 * n], i = sel[3 * n + 1], h = sel[3 * n + 2];
        if (b < 0 || b >= B || i < 0 || i >= n_q || h < 0 || h >= Hq) return -1;
        if (seq_len[b] < n_q || seq_base[b] < 0 || seq_base[b] + seq_len[b] > capacity) return -1;
    }
    attn_ctx c = {k_codes, k_scales, v_codes, v_scales, k_fp8 != 0, Hkv, D, capacity, gscale, q,
                  seq_base, seq_len, n_q, Hq, sm_scale, sel, out, 0};
    parallel_for(attn_item, &c, n_sel, nthreads);
    return c.status;
}
