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

// One thread per (row, K|V, group of 16) of KV head blockIdx.y. Every divisor of the
// index decomposition is a compile-time constant (head_dim is a template parameter;
// divisions by run-time values cost tens of instructions each). A row's D/16 groups of K
// (or of V) are D/16 consecutive threads, aligned, so K8V4's row-scaled FP8 K (KF = 1)
// reduces its row maximum across them; every such run of threads is active as a whole
// (the thread count is a multiple of D/16).
template <int D, int KF>
__global__ __launch_bounds__(256) void append_kernel(AppendParams p) {
    constexpr int groups = D / 16;
    const uint32_t tx = blockIdx.x * 256u + threadIdx.x;
    if (tx >= (uint32_t)(p.rows * 2 * groups)) return;
    const int h = blockIdx.y;
    const int j = tx % groups;
    const int kv = (tx / groups) & 1;                 // 0 = K, 1 = V
    const int64_t r = tx / (2 * groups);
    int b = 0;
#pragma unroll
    for (int s = 1; s < kMaxSeqs; ++s)
        if (s < p.B && r >= p.row_start[s]) b = s;
    const int64_t slot = p.dst_start[b] + (r - p.row_start[b]);

    const uint16_t *src = (kv ? p.v_new : p.k_new) + (r * p.Hkv + h) * D + 16 * j;
    const uint4 w0 = *reinterpret_cast<const uint4 *>(src);
    const uint4 w1 = *reinterpret_cast<const uint4 *>(src + 8);
    const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};

    const int64_t plane_row = (int64_t)h * p.cap + slot;
    if (KF == 1 && kv == 0) {
        store_fp8_group<D>(w, j, p.kc, p.ks, plane_row);
        return;
    }
    uint32_t packed[2];
    const uint32_t sc = quantize_group(w, p.gscale[(b * p.Hkv + h) * 2 + kv], packed);
    uint8_t *codes = (kv ? p.vc : p.kc) + plane_row * (D / 2) + 8 * j;
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
    if (p.rows == 0) return hipSuccess;
    const int64_t threads = p.rows * 2 * (p.D / 16);  // per KV head; < 2^31 (checked by the caller)
    const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)p.Hkv);
    if (p.D == 256 && !p.k_fp8)
        hipLaunchKernelGGL((append_kernel<256, 0>), grid, dim3(256), 0, s, p);
    else if (p.D == 256)
        hipLaunchKernelGGL((append_kernel<256, 1>), grid, dim3(256), 0, s, p);
    else if (p.D == 128 && !p.k_fp8)
        hipLaunchKernelGGL((append_kernel<128, 0>), grid, dim3(256), 0, s, p);
    else if (p.D == 128)
        hipLaunchKernelGGL((append_kernel<128, 1>), grid, dim3(256), 0, s, p);
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
