// Quantise-on-append and global-scale calibration kernels (gfx950). The group
// quantiser (format and exact rounding) is in quantize.h.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "internal.h"
#include "decode_common.h"
#include "quantize.h"

namespace nvfp4 {
namespace {

using namespace dev;

// Where one append item -- a (row, K|V, group of 16) of KV head h -- reads and writes.
// Items are numbered so that each wave holds one plane: wave v of a head covers rows
// RW (v / 2) .. RW (v / 2) + RW - 1 (RW = 64 / (D/16) rows) of K (v even) or V (v odd), one
// group per lane, a row's D/16 groups on consecutive lanes. Every divisor of the index
// decomposition is a compile-time constant (head_dim is a template parameter; divisions by
// run-time values cost tens of instructions each).
struct AppendItem {
    int j, kv, b;
    int64_t r, plane_row;
};

// One of two kernel-argument pointers by a per-lane selector, as a + (sel ? b - a : 0). A
// plain select of two argument fields compiles to a per-lane vector load of the chosen
// field (a memory round trip before every access through it); the difference, taken through
// empty asm, stays a scalar, and the result stays derived from a global pointer (global, not
// flat, memory instructions).
template <typename T>
__device__ inline T *pick(int sel, T *a, T *b) {
    int64_t d = (int64_t)((uintptr_t)b - (uintptr_t)a);
    asm("" : "+s"(d));
    return (T *)((const char *)a + (sel ? d : 0));
}

template <int D>
__device__ inline AppendItem append_item(const AppendParams &p, uint32_t tx, int h) {
    constexpr int groups = D / 16, RW = 64 / groups;
    AppendItem it;
    const uint32_t lane = tx % 64, wv = tx / 64;
    it.j = lane % groups;
    it.kv = wv & 1;                                   // 0 = K, 1 = V
    it.r = (int64_t)(wv >> 1) * RW + lane / groups;
    // The sequence of row r (uniform loop over the sequences' scalar starts).
    it.b = 0;
    int64_t start = p.row_start[0], dst = p.dst_start[0];
    for (int s = 1; s < p.B; ++s) {
        const int64_t rs = p.row_start[s], ds = p.dst_start[s];
        if (it.r >= rs) {
            it.b = s;
            start = rs;
            dst = ds;
        }
    }
    it.plane_row = (int64_t)h * p.cap + dst + (it.r - start);
    return it;
}

template <int D>
__device__ inline void load_item(const AppendParams &p, const AppendItem &it, int h, uint32_t (&w)[8]) {
    const uint16_t *src = pick(it.kv, p.k_new, p.v_new) + (it.r * p.Hkv + h) * D + 16 * it.j;
    const uint4 w0 = *reinterpret_cast<const uint4 *>(src);
    const uint4 w1 = *reinterpret_cast<const uint4 *>(src + 8);
    w[0] = w0.x; w[1] = w0.y; w[2] = w0.z; w[3] = w0.w;
    w[4] = w1.x; w[5] = w1.y; w[6] = w1.z; w[7] = w1.w;
}

// One thread per item of KV head blockIdx.y (quantisers in quantize.h). A wave holds one
// plane, so K8V4's two quantisers (KF = 1) never share a wave; its row-scaled FP8 K reduces
// the row maximum across the row's D/16 lanes (a row's lanes are all active or all not).
template <int D, int KF>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    constexpr int groups = D / 16;
    const int h = blockIdx.y;
    const uint32_t tx = blockIdx.x * 256u + threadIdx.x;
    const AppendItem it = append_item<D>(p, tx, h);
    if (it.r >= p.rows) return;
    uint32_t w[8];
    load_item<D>(p, it, h, w);
    if (KF == 1 && it.kv == 0) {
        uint32_t am = amax16_bits(w);
#pragma unroll
        for (int off = 1; off < groups; off <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
        const float s = fp8_row_scale(am);
        uint32_t c[4];
        fp8_row_codes(w, s, c);
        *reinterpret_cast<uint4 *>(p.kc + it.plane_row * D + 16 * it.j) = make_uint4(c[0], c[1], c[2], c[3]);
        if (it.j == 0) reinterpret_cast<float *>(p.ks)[it.plane_row] = s;
        return;
    }
    uint32_t packed[2];
    const uint32_t sc = quantize_group(w, p.gscale[(it.b * p.Hkv + h) * 2 + it.kv], packed);
    *reinterpret_cast<uint2 *>(pick(it.kv, p.kc, p.vc) + it.plane_row * (D / 2) + 8 * it.j) =
        make_uint2(packed[0], packed[1]);
    pick(it.kv, p.ks, p.vs)[it.plane_row * groups + it.j] = (uint8_t)sc;
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
    if (p.rows == 0) return hipSuccess;
    // per KV head: a pair of waves (K, V) per 64 / (D/16) rows; < 2^31 (rows * D/8 is
    // checked by the caller)
    const int64_t rw = 64 / (p.D / 16);
    const int64_t threads = (p.rows + rw - 1) / rw * 128;
    const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)p.Hkv);
    const dim3 block(256);
    if (p.D == 256 && !p.k_fp8)
        hipLaunchKernelGGL((append_kernel<256, 0>), grid, block, 0, s, p);
    else if (p.D == 256)
        hipLaunchKernelGGL((append_kernel<256, 1>), grid, block, 0, s, p);
    else if (p.D == 128 && !p.k_fp8)
        hipLaunchKernelGGL((append_kernel<128, 0>), grid, block, 0, s, p);
    else if (p.D == 128)
        hipLaunchKernelGGL((append_kernel<128, 1>), grid, block, 0, s, p);
    else
        return hipErrorInvalidValue;
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
