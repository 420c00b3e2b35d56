// Streaming-read probe: the HBM read rate one plain kernel reaches on this device, the
// practical ceiling that the decode kernels' bandwidth is judged against (knoopx/ninfer
// page, "Quick start": the engine ships a standalone HBM probe next to its build).
//
// Each thread reads 16-byte words in a grid-stride loop, four independent loads in flight
// per trip, with the streaming (non-temporal) cache policy that the decode kernels' KV loads
// use (on MI355X it reads about 11% faster than the default policy), and folds them into one
// word; each workgroup writes one word of the sink, so
// the reads cannot be dropped and the writes are negligible.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"

namespace nvfp4 {
namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;

constexpr int kProbeThreads = 256;
constexpr int kUnroll = 4;

// One raw buffer per window of just under 2 GiB (buffer offsets are 32-bit); an offset past
// the window's end is answered with zeros and no memory access.
__global__ __launch_bounds__(kProbeThreads) void read_probe_kernel(const uint8_t *buf, uint64_t words,
                                                                   uint32_t *sink) {
    constexpr uint64_t kWindowWords = ((uint64_t)1 << 27) - 16;     // 16-byte words, below 2^31 bytes
    const uint64_t stride = (uint64_t)gridDim.x * kProbeThreads;
    uint32_t acc = 0;
    for (uint64_t w0 = 0; w0 < words; w0 += kWindowWords) {
        const uint64_t n = words - w0 < kWindowWords ? words - w0 : kWindowWords;
        const rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(buf) + w0 * 16, (short)0,
                                                           (int)(n * 16), 0x00020000);
        for (uint64_t i = (uint64_t)blockIdx.x * kProbeThreads + threadIdx.x; i < n; i += kUnroll * stride) {
            u32x4_t v[kUnroll];
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) {
                const uint64_t j = i + k * stride;
                // j < n keeps the offset below 2^31; past n the load is answered with zeros
                const uint32_t off = j < n ? (uint32_t)(j * 16) : 0x80000000u;
                v[k] = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);   // nt
            }
#pragma unroll
            for (int k = 0; k < kUnroll; ++k) acc ^= v[k][0] ^ v[k][1] ^ v[k][2] ^ v[k][3];
        }
    }
    __shared__ uint32_t part[kProbeThreads / 64];
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

hipError_t launch_read_probe(const void *buf, uint64_t bytes, uint32_t *sink, int workgroups, hipStream_t s) {
    hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s,
                       static_cast<const uint8_t *>(buf), bytes / 16, sink);
    return hipGetLastError();
}

}  // namespace nvfp4
