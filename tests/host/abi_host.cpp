// Host-only build of the C ABI's argument validation (quantized_kv_decode_amd/csrc/api.cpp)
// for sanitizer runs: the kernel launchers are replaced by stubs that count their calls, so
// every call below either fails validation (and must launch nothing) or reaches a stub.
// Built with g++ -fsanitize=address,undefined by tests/test_sanitizers.py; exits non-zero on
// the first wrong return code.
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "internal.h"
#include "nvfp4_kv.h"

static int g_launches = 0;
const char *hipGetErrorString(hipError_t) { return "stub"; }
namespace nvfp4 {
hipError_t launch_calibrate(const CalibParams &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_append(const AppendParams &, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_partial(const DecodeParams &, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_pair(const DecodeParams &, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_decode_combine(const DecodeParams &, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_read_probe(const void *, uint64_t, uint32_t *, int, hipStream_t) { ++g_launches; return hipSuccess; }
}  // namespace nvfp4

static int failures = 0;
#define EXPECT(call, code, launches)                                                                  \
    do {                                                                                              \
        const int before = g_launches;                                                                \
        const int rc = (call);                                                                        \
        if (rc != (code) || g_launches - before != (launches)) {                                      \
            std::printf("FAIL line %d: rc %d (want %d), launches %d (want %d): %s\n", __LINE__, rc,   \
                        (code), g_launches - before, (launches), nvfp4_last_error());                 \
            ++failures;                                                                               \
        }                                                                                             \
    } while (0)

static void *P(uintptr_t a) { return reinterpret_cast<void *>(a); }

int main() {
    nvfp4_kv_cache c;
    std::memset(&c, 0, sizeof c);
    c.k_codes = P(0x100000); c.k_scales = P(0x110000); c.v_codes = P(0x120000); c.v_scales = P(0x130000);
    c.num_kv_heads = 4; c.head_dim = 256; c.capacity = 100000; c.kv_format = NVFP4_KV_NVFP4;
    const int64_t base0[1] = {0}, len100[1] = {100}, len0[1] = {0}, big[1] = {200000};
    float *g = static_cast<float *>(P(0x400000));
    void *q = P(0x200000), *out = P(0x300000), *ws = P(0x500000), *kn = P(0x600000);

    // decode: valid call launches partial + combine; each invalid argument launches nothing
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 1, base0, len100, 1, 24, 0.0625f, ws, 1 << 30, nullptr), 0, 2);
    EXPECT(nvfp4_decode_attn(nullptr, g, q, out, 0, 1, base0, len100, 1, 24, 0.0625f, ws, 1 << 30, nullptr), NVFP4_EINVAL, 0);
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 1, base0, len0, 1, 24, 0.0625f, ws, 1 << 30, nullptr), NVFP4_ERANGE, 0);
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 1, base0, big, 1, 24, 0.0625f, ws, 1 << 30, nullptr), NVFP4_ERANGE, 0);
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 1, base0, len100, 1, 25, 0.0625f, ws, 1 << 30, nullptr), NVFP4_EUNSUPPORTED, 0);
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 9, base0, len100, 1, 24, 0.0625f, ws, 1 << 30, nullptr), NVFP4_EUNSUPPORTED, 0);
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 7, 1, base0, len100, 1, 24, 0.0625f, ws, 1 << 30, nullptr), NVFP4_EINVAL, 0);
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 1, base0, len100, 1, 24, 0.0625f, ws, 16, nullptr), NVFP4_EWORKSPACE, 0);
    EXPECT(nvfp4_decode_attn(&c, g, P(0x200008), out, 0, 1, base0, len100, 1, 24, 0.0625f, ws, 1 << 30, nullptr), NVFP4_EINVAL, 0);
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 1, base0, len100, 1, 24, 1.0f / 0.0f, ws, 1 << 30, nullptr), NVFP4_EINVAL, 0);
    // every sequence count and a spread of lengths, n_q and head counts through the planner
    int64_t lens[8], bases[8];
    for (int B = 1; B <= 8; ++B)
        for (int nq = 1; nq <= 300; nq += 37)
            for (int64_t L = nq; L < 90000; L = L * 3 + 7) {
                for (int b = 0; b < B; ++b) { lens[b] = L + b; bases[b] = 0; }
                c.capacity = L + 8;
                const size_t need = nvfp4_decode_attn_workspace_bytes(&c, B, lens, nq, 24);
                EXPECT(nvfp4_decode_step(&c, g, kn, kn, q, out, 0, B, bases, lens, nq, 24, 0.0625f, ws, need, nullptr),
                       (6 * nq > 8192) ? NVFP4_EUNSUPPORTED : 0, (6 * nq > 8192) ? 0 : (6 * nq > 128 ? 3 : 2));
                EXPECT(nvfp4_decode_step(&c, g, kn, kn, q, out, 0, B, bases, lens, nq, 24, 0.0625f, ws, need ? need - 1 : 0,
                                         nullptr), (6 * nq > 8192) ? NVFP4_EUNSUPPORTED : NVFP4_EWORKSPACE, 0);
            }
    c.capacity = 100000;
    // K8V4 and invalid formats
    c.kv_format = NVFP4_KV_K8V4;
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 1, base0, len100, 1, 24, 0.0625f, ws, 1 << 30, nullptr), 0, 2);
    c.kv_format = 5;
    EXPECT(nvfp4_decode_attn(&c, g, q, out, 0, 1, base0, len100, 1, 24, 0.0625f, ws, 1 << 30, nullptr), NVFP4_EINVAL, 0);
    c.kv_format = NVFP4_KV_NVFP4;
    // append and calibrate
    const int64_t wp[1] = {10}, nn[1] = {5}, nneg[1] = {-1}, wpfar[1] = {99998};
    EXPECT(nvfp4_kv_append(&c, kn, kn, g, 1, base0, wp, nn, nullptr), 0, 1);
    EXPECT(nvfp4_kv_append(&c, kn, kn, g, 1, base0, wpfar, nn, nullptr), NVFP4_ERANGE, 0);
    EXPECT(nvfp4_kv_append(&c, kn, kn, g, 1, base0, wp, nneg, nullptr), NVFP4_EINVAL, 0);
    EXPECT(nvfp4_kv_append(&c, nullptr, nullptr, g, 1, base0, wp, len0, nullptr), 0, 0);
    EXPECT(nvfp4_kv_calibrate(&c, kn, kn, 1, nn, g, nullptr), 0, 1);
    EXPECT(nvfp4_kv_calibrate(&c, kn, kn, 1, nneg, g, nullptr), NVFP4_EINVAL, 0);
    // device-length step and the probe
    EXPECT(nvfp4_decode_step_dev_len(&c, g, kn, kn, q, out, 0, 1, base0, len100, static_cast<int64_t *>(P(0x700000)), 1,
                                     24, 0.0625f, ws, 1 << 30, nullptr), 0, 2);
    EXPECT(nvfp4_decode_step_dev_len(&c, g, kn, kn, q, out, 0, 1, base0, len100, static_cast<int64_t *>(P(0x700004)), 1,
                                     24, 0.0625f, ws, 1 << 30, nullptr), NVFP4_EINVAL, 0);
    EXPECT(nvfp4_hbm_read_probe(P(0x800000), 4096, P(0x900000), 8, nullptr), 0, 1);
    EXPECT(nvfp4_hbm_read_probe(P(0x800000), 4095, P(0x900000), 8, nullptr), NVFP4_EINVAL, 0);
    std::printf("abi host checks: %d failures, %d launches\n", failures, g_launches);
    return failures ? 1 : 0;
}
