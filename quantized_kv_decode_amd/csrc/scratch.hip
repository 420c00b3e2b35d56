// The decode step for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation): the same step as
// nvfp4_decode_step, with its split-K partials in a fixed device array instead of a
// caller-provided workspace.
//
// The array lives in this file; every GPU the library runs on holds its own copy until the
// process ends. Its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) on the first call there and kept; host code only ever passes that
// address on, never the array's own name (which on the host is a stand-in, not a device
// address). Calls that overlap on one GPU share the array and race; calls on one stream
// are ordered. The kernels overwrite every part of it they later read, so nothing needs
// clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "nvfp4_kv.h"

namespace {

constexpr size_t kScratchBytes = (size_t)NVFP4_NOALLOC_SCRATCH_MIB << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];

// Device address of this device's scratch array (looked up once per device), or an
// NVFP4 error code.
int scratch_for_current_device(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return nvfp4::report_error(NVFP4_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return nvfp4::report_error(NVFP4_EHIP, "device %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return nvfp4::report_error(NVFP4_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev,
                                       hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return NVFP4_OK;
}

}  // namespace

extern "C" int nvfp4_decode_step_noalloc(const nvfp4_kv_cache *cache, const float *global_scale,
                                         const void *k_new, const void *v_new, const void *q, void *out,
                                         int32_t out_dtype, int32_t num_seqs, const int64_t *seq_base,
                                         const int64_t *seq_len, int32_t n_q, int32_t num_q_heads,
                                         float sm_scale, void *stream) {
    // Size first (host only): a shape whose partials do not fit is rejected before any HIP call.
    const size_t need = nvfp4_decode_attn_workspace_bytes(cache, num_seqs, seq_len, n_q, num_q_heads);
    if (need == 0)   // invalid arguments: the step's own validation reports which
        return nvfp4_decode_step(cache, global_scale, k_new, v_new, q, out, out_dtype, num_seqs, seq_base,
                                 seq_len, n_q, num_q_heads, sm_scale, nullptr, 0, stream);
    if (need > kScratchBytes)
        return nvfp4::report_error(NVFP4_EWORKSPACE, "this step needs %zu bytes of partials; the static scratch "
                                   "holds %zu (use nvfp4_decode_step with a workspace)", need, kScratchBytes);
    void *ws = nullptr;
    const int rc = scratch_for_current_device(&ws);
    if (rc != NVFP4_OK) return rc;
    return nvfp4_decode_step(cache, global_scale, k_new, v_new, q, out, out_dtype, num_seqs, seq_base, seq_len,
                             n_q, num_q_heads, sm_scale, ws, kScratchBytes, stream);
}
