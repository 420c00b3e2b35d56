// Quantise-on-append and global-scale calibration kernels (gfx950).
//
// Format (gzenz/ninfer page, "Context and model", NVFP4 KV cache bullet): 4-bit
// E2M1 codes, two per byte, with one E4M3 scale per 16 elements; here also a
// per-(sequence, KV head) fp32 global scale g = amax / 2688.
//
// Rounding is decided on exact reals. The group scale is the E4M3 value nearest
// amax/(6g) (ties to the even code, saturating at 448); each element's magnitude
// is the E2M1 value nearest |x|/(S g) (ties to the even code, saturating at 6).
// How the kernel makes those decisions exact:
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
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "internal.h"

namespace nvfp4 {
namespace {

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

// Magnitude code of a bf16 magnitude a16 given the group's seven thresholds:
// u[k] <-> midpoint k in (0.25 >, 0.75 >=, 1.25 >, 1.75 >=, 2.5 >, 3.5 >=, 5 >).
__device__ inline uint32_t e2m1_mag(uint32_t a16, const uint32_t u[7]) {
    const uint32_t c1 = a16 > u[3];
    const uint32_t c2 = a16 > (c1 ? u[5] : u[1]);
    const uint32_t t3 = c1 ? (c2 ? u[6] : u[4]) : (c2 ? u[2] : u[0]);
    const uint32_t c3 = a16 > t3;
    return (c1 << 2) | (c2 << 1) | c3;
}

// One thread per (row, head, K|V, group of 16).
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    const int groups = p.D / 16;
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t per_kv = p.rows * p.Hkv * groups;
    if (tid >= 2 * per_kv) return;
    const int kv = tid >= per_kv;                     // 0 = K, 1 = V
    const int64_t t = tid - kv * per_kv;
    const int j = (int)(t % groups);
    const int h = (int)((t / groups) % p.Hkv);
    const int64_t r = t / ((int64_t)groups * p.Hkv);
    int b = 0;
#pragma unroll
    for (int s = 1; s < kMaxSeqs; ++s)
        if (s < p.B && r >= p.row_start[s]) b = s;
    const int64_t slot = p.dst_start[b] + (r - p.row_start[b]);

    const uint16_t *src = (kv ? p.v_new : p.k_new) + (r * p.Hkv + h) * p.D + 16 * j;
    const uint4 w0 = *reinterpret_cast<const uint4 *>(src);
    const uint4 w1 = *reinterpret_cast<const uint4 *>(src + 8);
    const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};

    uint32_t amax16 = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        amax16 = max(amax16, w[k] & 0x7FFFu);
        amax16 = max(amax16, (w[k] >> 16) & 0x7FFFu);
    }
    const double g = (double)p.gscale[(b * p.Hkv + h) * 2 + kv];
    const double amax = (double)__builtin_bit_cast(float, amax16 << 16);
    int sc = 0;
    if (g > 0.0 && amax > 0.0) sc = e4m3_code_exact(amax, 6.0 * g);
    const double Sg = e4m3_pos_value(sc) * g;        // exact (<= 28 significant bits)

    uint32_t u[7];
    if (Sg > 0.0) {
        u[0] = thr_gt(0.25 * Sg); u[1] = thr_ge(0.75 * Sg); u[2] = thr_gt(1.25 * Sg);
        u[3] = thr_ge(1.75 * Sg); u[4] = thr_gt(2.5 * Sg);  u[5] = thr_ge(3.5 * Sg);
        u[6] = thr_gt(5.0 * Sg);
    } else {
#pragma unroll
        for (int k = 0; k < 7; ++k) u[k] = 0xFFFFu;  // every magnitude 0
    }

    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t lo = w[k] & 0xFFFFu, hi = w[k] >> 16;
        const uint32_t c0 = e2m1_mag(lo & 0x7FFFu, u) | ((lo >> 12) & 8u);
        const uint32_t c1 = e2m1_mag(hi & 0x7FFFu, u) | ((hi >> 12) & 8u);
        packed[k >> 2] |= (c0 | (c1 << 4)) << (8 * (k & 3));
    }
    const int64_t plane_row = (int64_t)h * p.cap + slot;
    uint8_t *codes = (kv ? p.vc : p.kc) + plane_row * (p.D / 2) + 8 * j;
    *reinterpret_cast<uint2 *>(codes) = make_uint2(packed[0], packed[1]);
    (kv ? p.vs : p.ks)[plane_row * groups + j] = (uint8_t)sc;
}

// ---- calibration: g[b][h][kv] = fp32(amax / 2688) ------------------------------------
__global__ __launch_bounds__(64) void calib_init_kernel(uint32_t *g, int n) {
    const int i = blockIdx.x * 64 + threadIdx.x;
    if (i < n) g[i] = 0u;
}

// grid.y = B * Hkv * 2 (b, h, kv); grid.x strides over that slice's 16-byte chunks.
__global__ __launch_bounds__(256) void calib_reduce_kernel(CalibParams p) {
    const int slice = blockIdx.y;
    const int kv = slice & 1, h = (slice >> 1) % p.Hkv, b = (slice >> 1) / p.Hkv;
    const int64_t r0 = p.row_start[b], nrows = p.row_start[b + 1] - r0;
    const int cpr = p.D / 8;                          // 16-byte chunks per row
    const int64_t nchunks = nrows * cpr;
    const uint16_t *base = (kv ? p.v_rows : p.k_rows);
    uint32_t m = 0;
    for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < nchunks; c += (int64_t)gridDim.x * 256) {
        const int64_t r = r0 + c / cpr;
        const uint4 v = *reinterpret_cast<const uint4 *>(base + (r * p.Hkv + h) * p.D + 8 * (c % cpr));
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) m = max(m, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
    }
    // Non-negative floats order like their bit patterns, so the max is an integer max
    // (order-independent, hence deterministic).
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
    __shared__ uint32_t part[4];
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        m = max(max(part[0], part[1]), max(part[2], part[3]));
        if (m) atomicMax(reinterpret_cast<uint32_t *>(p.gscale) + slice, m << 16);
    }
}

__global__ __launch_bounds__(64) void calib_finalize_kernel(float *g, int n) {
    const int i = blockIdx.x * 64 + threadIdx.x;
    if (i < n) {
        // The fp64 quotient rounded to fp32 is the correctly rounded fp32 quotient.
        const double amax = (double)__builtin_bit_cast(float, reinterpret_cast<uint32_t *>(g)[i]);
        g[i] = (float)(amax / 2688.0);
    }
}

}  // namespace

hipError_t launch_append(const AppendParams &p, hipStream_t s) {
    const int64_t threads = 2 * p.rows * p.Hkv * (p.D / 16);
    if (threads == 0) return hipSuccess;
    const int64_t blocks = (threads + 255) / 256;
    hipLaunchKernelGGL(append_kernel, dim3((unsigned)blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_calibrate(const CalibParams &p, hipStream_t s) {
    const int n = p.B * p.Hkv * 2;
    hipLaunchKernelGGL(calib_init_kernel, dim3((n + 63) / 64), dim3(64), 0, s,
                       reinterpret_cast<uint32_t *>(p.gscale), n);
    int64_t maxrows = 0;
    for (int b = 0; b < p.B; ++b) maxrows = std::max(maxrows, p.row_start[b + 1] - p.row_start[b]);
    const int64_t chunks = maxrows * (p.D / 8);
    int64_t gx = (chunks + 255) / 256;
    if (gx > 256) gx = 256;
    if (gx < 1) gx = 1;
    hipLaunchKernelGGL(calib_reduce_kernel, dim3((unsigned)gx, (unsigned)n), dim3(256), 0, s, p);
    hipLaunchKernelGGL(calib_finalize_kernel, dim3((n + 63) / 64), dim3(64), 0, s, p.gscale, n);
    return hipGetLastError();
}

}  // namespace nvfp4
