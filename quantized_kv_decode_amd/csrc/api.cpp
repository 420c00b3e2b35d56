// Host side of the C ABI: argument validation, split-K planning and launches.
// No allocation, no synchronisation: every call enqueues on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdint>
#include <cstring>
#include <string>

#include "internal.h"
#include "nvfp4_kv.h"

namespace {
thread_local std::string g_last_error;
}  // namespace

namespace nvfp4 {
int report_error(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}
}  // namespace nvfp4

namespace {

int (*const fail)(int, const char *, ...) = &nvfp4::report_error;

int ok() {
    g_last_error.clear();
    return NVFP4_OK;
}

bool aligned16(const void *p) { return p && (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_cache(const nvfp4_kv_cache *c) {
    if (!c) return fail(NVFP4_EINVAL, "cache is null");
    if (!aligned16(c->k_codes) || !aligned16(c->k_scales) || !aligned16(c->v_codes) || !aligned16(c->v_scales))
        return fail(NVFP4_EINVAL, "pool planes must be non-null and 16-byte aligned");
    if (c->num_kv_heads < 1) return fail(NVFP4_EINVAL, "num_kv_heads must be >= 1");
    if (c->capacity < 1) return fail(NVFP4_EINVAL, "capacity must be >= 1");
    if (c->kv_format != NVFP4_KV_NVFP4 && c->kv_format != NVFP4_KV_K8V4)
        return fail(NVFP4_EINVAL, "kv_format %d invalid (NVFP4_KV_NVFP4 or NVFP4_KV_K8V4)", c->kv_format);
    if (c->head_dim != 128 && c->head_dim != 256)
        return fail(NVFP4_EUNSUPPORTED, "head_dim %d unsupported (128 or 256)", c->head_dim);
    // kernels address one head plane with 32-bit byte offsets (K8V4's K codes: head_dim bytes a row)
    const int64_t row_bytes = c->kv_format == NVFP4_KV_K8V4 ? c->head_dim : c->head_dim / 2;
    if (c->capacity > (int64_t)INT32_MAX / row_bytes)
        return fail(NVFP4_EUNSUPPORTED, "capacity %lld too large: a head's code plane must stay below 2^31 bytes",
                    (long long)c->capacity);
    return NVFP4_OK;
}

int check_seqs(int32_t num_seqs) {
    if (num_seqs < 1) return fail(NVFP4_EINVAL, "num_seqs must be >= 1");
    if (num_seqs > NVFP4_MAX_SEQS) return fail(NVFP4_EUNSUPPORTED, "num_seqs %d > %d", num_seqs, NVFP4_MAX_SEQS);
    return NVFP4_OK;
}

int hip_status(hipError_t e, const char *what) {
    if (e != hipSuccess) return fail(NVFP4_EHIP, "%s: %s", what, hipGetErrorString(e));
    return ok();
}

// Validates the decode shape and fills the split plan. Returns an NVFP4 code.
int make_plan(const nvfp4_kv_cache *c, int32_t num_seqs, const int64_t *seq_base, const int64_t *seq_len,
              int32_t n_q, int32_t num_q_heads, nvfp4::SplitPlan &pl) {
    int rc = check_cache(c);
    if (rc) return rc;
    if ((rc = check_seqs(num_seqs))) return rc;
    if (!seq_len) return fail(NVFP4_EINVAL, "seq_len is null");
    if (n_q < 1) return fail(NVFP4_EINVAL, "n_q must be >= 1");
    if (num_q_heads < 1) return fail(NVFP4_EINVAL, "num_q_heads must be >= 1");
    if (num_q_heads % c->num_kv_heads != 0)
        return fail(NVFP4_EUNSUPPORTED, "num_q_heads %d not a multiple of num_kv_heads %d", num_q_heads,
                    c->num_kv_heads);
    const int G = num_q_heads / c->num_kv_heads;
    if ((int64_t)G * n_q > NVFP4_MAX_ROWS)
        return fail(NVFP4_EUNSUPPORTED, "GQA group %d x n_q %d = %d rows > %d", G, n_q, G * n_q, NVFP4_MAX_ROWS);
    for (int b = 0; b < num_seqs; ++b) {
        if (seq_len[b] < n_q) return fail(NVFP4_ERANGE, "seq_len[%d] = %lld < n_q", b, (long long)seq_len[b]);
        if (seq_len[b] > c->capacity) return fail(NVFP4_ERANGE, "seq_len[%d] past capacity", b);
        if (seq_base) {
            if (seq_base[b] < 0 || seq_base[b] + seq_len[b] > c->capacity)
                return fail(NVFP4_ERANGE, "sequence %d slots [%lld, %lld) outside the pool", b,
                            (long long)seq_base[b], (long long)(seq_base[b] + seq_len[b]));
        }
    }
    pl.B = num_seqs;
    pl.Hkv = c->num_kv_heads;
    pl.Hq = num_q_heads;
    pl.G = G;
    pl.n_q = n_q;
    pl.R = G * n_q;
    // Up to 64 rows per KV head go through the decode kernels in one pass; more (wide draft
    // windows, prefill chunks) are cut into 32-row chunks that run side by side as grid y of
    // one launch over the same units, with correspondingly fewer units. 32-row chunks run on
    // the single-wave-per-block kernel: against 64-row chunks on the wave-pair kernel, 96
    // rows over 131k tokens 107.8 -> 91.2 us, a 1,024-token prefill chunk into 32k tokens
    // (6,144 rows) 1,342 -> 923 us; 48-row chunks 1,040 us.
    pl.chunk_rows = pl.R <= nvfp4::kMaxRows ? pl.R : nvfp4::kChunkRows;
    pl.chunks = (pl.R + pl.chunk_rows - 1) / pl.chunk_rows;
    pl.NT = (std::min(pl.chunk_rows, pl.R) + 15) / 16;
    pl.D = c->head_dim;
    // Fill every CU with decode_units_per_cu(NT) units. Splits go greedily to the sequence
    // whose units are currently longest, so ragged batches get near-equal units.
    const int64_t grid_y = pl.chunks;
    const int64_t slots = std::max<int64_t>((int64_t)nvfp4::kCUs * nvfp4::decode_units_per_cu(pl.NT) / grid_y,
                                            (int64_t)num_seqs * pl.Hkv);
    int64_t nsp[nvfp4::kMaxSeqs];
    for (int b = 0; b < num_seqs; ++b) nsp[b] = 1;
    int64_t total = (int64_t)num_seqs * pl.Hkv;
    const int64_t min_len = 4 * nvfp4::kBlockTokens;     // at least one block per wave
    for (;;) {
        int best = -1;
        double best_len = 0;
        for (int b = 0; b < num_seqs; ++b) {
            const double len = (double)seq_len[b] / (double)nsp[b];
            if (len > best_len) { best_len = len; best = b; }
        }
        if (best < 0 || total + pl.Hkv > slots) break;
        if ((double)seq_len[best] / (double)(nsp[best] + 1) < (double)min_len) break;
        nsp[best] += 1;
        total += pl.Hkv;
    }
    // No unit longer than kMaxUnitTokens (the fp16 probability floor, see internal.h), even if
    // that takes more units than resident workgroup slots (very many sequence x head pairs).
    for (int b = 0; b < num_seqs; ++b)
        nsp[b] = std::max<int64_t>(nsp[b], (seq_len[b] + nvfp4::kMaxUnitTokens - 1) / nvfp4::kMaxUnitTokens);
    int32_t ub = 0;
    for (int b = 0; b < num_seqs; ++b) {
        int64_t len = (seq_len[b] + nsp[b] - 1) / nsp[b];
        len = (len + nvfp4::kBlockTokens - 1) / nvfp4::kBlockTokens * nvfp4::kBlockTokens;
        int64_t ns = (seq_len[b] + len - 1) / len;
        // The last unit must hold the n_q newest tokens (a decode step appends them in
        // the workgroup that reads them): a shorter remainder joins the unit before it.
        if (ns > 1 && seq_len[b] - (ns - 1) * len < n_q) ns -= 1;
        pl.split_len[b] = (int32_t)len;
        pl.n_split[b] = (int32_t)ns;
        pl.unit_base[b] = ub;
        ub += (int32_t)(ns * pl.Hkv);
    }
    for (int b = num_seqs; b < nvfp4::kMaxSeqs; ++b) {
        pl.split_len[b] = 0;
        pl.n_split[b] = 0;
        pl.unit_base[b] = ub;
    }
    pl.units = ub;
    return NVFP4_OK;
}

size_t workspace_for(const nvfp4::SplitPlan &pl) {
    // o: units x R x D floats, then m and l: units x R floats each, each part 256-byte aligned.
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t ur = (size_t)pl.units * pl.R;
    return al(ur * pl.D * sizeof(float)) + 2 * al(ur * sizeof(float));
}

void fill_decode(nvfp4::DecodeParams &dp, const nvfp4::SplitPlan &pl, const nvfp4_kv_cache *c,
                 const float *global_scale, const void *q, const int64_t *seq_base, const int64_t *seq_len,
                 float sm_scale, void *workspace) {
    std::memset(&dp, 0, sizeof dp);
    dp.kc = static_cast<uint8_t *>(c->k_codes);
    dp.ks = static_cast<uint8_t *>(c->k_scales);
    dp.vc = static_cast<uint8_t *>(c->v_codes);
    dp.vs = static_cast<uint8_t *>(c->v_scales);
    dp.cap = c->capacity;
    dp.k_fp8 = c->kv_format == NVFP4_KV_K8V4;
    dp.gscale = global_scale;
    dp.q = static_cast<const uint16_t *>(q);
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    const size_t ur = (size_t)pl.units * pl.R;
    char *ws = static_cast<char *>(workspace);
    dp.ws_o = reinterpret_cast<float *>(ws);
    dp.ws_m = reinterpret_cast<float *>(ws + al(ur * pl.D * sizeof(float)));
    dp.ws_l = reinterpret_cast<float *>(ws + al(ur * pl.D * sizeof(float)) + al(ur * sizeof(float)));
    dp.sm_scale = sm_scale;
    dp.B = pl.B;
    dp.Hkv = pl.Hkv;
    dp.Hq = pl.Hq;
    dp.G = pl.G;
    dp.n_q = pl.n_q;
    dp.R = pl.R;
    dp.row0 = 0;
    dp.Rc = std::min(pl.chunk_rows, pl.R);
    dp.grid_y = 1;
    for (int b = 0; b < nvfp4::kMaxSeqs; ++b) {
        dp.seq_base[b] = (b < pl.B && seq_base) ? seq_base[b] : 0;
        dp.seq_len[b] = (b < pl.B) ? seq_len[b] : 0;
        dp.n_split[b] = pl.n_split[b];
        dp.split_len[b] = pl.split_len[b];
        dp.unit_base[b] = pl.unit_base[b];
    }
    dp.units = pl.units;
}

// The partial kernel over every row chunk: one launch, the chunks on grid y over the same
// units. Up to kMaxStoreRows rows, the workgroup of each sequence's last unit in every
// chunk stores the step's new rows before reading them (the chunks store identical bytes,
// and each workgroup orders its own stores before its loads); above that the caller has
// stored them with the append kernel.
hipError_t launch_partials(nvfp4::DecodeParams dp, const nvfp4::SplitPlan &pl, hipStream_t s) {
    dp.row0 = 0;
    dp.Rc = pl.chunk_rows;
    dp.grid_y = pl.chunks;
    if (pl.R > nvfp4::kMaxStoreRows) dp.k_new = dp.v_new = nullptr;
    return nvfp4::launch_decode_partial(dp, pl.D, pl.NT, s);
}

int check_decode_common(const float *global_scale, void *workspace, size_t workspace_bytes,
                        const nvfp4::SplitPlan &pl) {
    if (!aligned16(global_scale)) return fail(NVFP4_EINVAL, "global_scale must be non-null and 16-byte aligned");
    if (!aligned16(workspace)) return fail(NVFP4_EINVAL, "workspace must be non-null and 16-byte aligned");
    const size_t need = workspace_for(pl);
    if (workspace_bytes < need)
        return fail(NVFP4_EWORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
    return NVFP4_OK;
}

}  // namespace

extern "C" {

const char *nvfp4_last_error(void) { return g_last_error.c_str(); }

int nvfp4_kv_calibrate(const nvfp4_kv_cache *cache, const void *k_rows, const void *v_rows, int32_t num_seqs,
                       const int64_t *n_rows, float *global_scale, void *stream) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = check_seqs(num_seqs))) return rc;
    if (!n_rows) return fail(NVFP4_EINVAL, "n_rows is null");
    if (!aligned16(global_scale)) return fail(NVFP4_EINVAL, "global_scale must be non-null and 16-byte aligned");
    nvfp4::CalibParams p;
    std::memset(&p, 0, sizeof p);
    int64_t acc = 0;
    for (int b = 0; b < num_seqs; ++b) {
        if (n_rows[b] < 0) return fail(NVFP4_EINVAL, "n_rows[%d] < 0", b);
        p.row_start[b] = acc;
        acc += n_rows[b];
    }
    for (int b = num_seqs; b <= nvfp4::kMaxSeqs; ++b) p.row_start[b] = acc;
    if (acc > 0 && (!aligned16(k_rows) || !aligned16(v_rows)))
        return fail(NVFP4_EINVAL, "k_rows/v_rows must be non-null and 16-byte aligned");
    p.k_rows = static_cast<const uint16_t *>(k_rows);
    p.v_rows = static_cast<const uint16_t *>(v_rows);
    p.gscale = global_scale;
    p.B = num_seqs;
    p.Hkv = cache->num_kv_heads;
    p.D = cache->head_dim;
    return hip_status(nvfp4::launch_calibrate(p, static_cast<hipStream_t>(stream)), "calibrate launch");
}

int nvfp4_kv_append(const nvfp4_kv_cache *cache, const void *k_new, const void *v_new, const float *global_scale,
                    int32_t num_seqs, const int64_t *seq_base, const int64_t *write_pos, const int64_t *n_new,
                    void *stream) {
    int rc = check_cache(cache);
    if (rc) return rc;
    if ((rc = check_seqs(num_seqs))) return rc;
    if (!seq_base || !write_pos || !n_new) return fail(NVFP4_EINVAL, "seq_base/write_pos/n_new must be non-null");
    if (!aligned16(global_scale)) return fail(NVFP4_EINVAL, "global_scale must be non-null and 16-byte aligned");
    nvfp4::AppendParams p;
    std::memset(&p, 0, sizeof p);
    int64_t acc = 0;
    for (int b = 0; b < num_seqs; ++b) {
        if (n_new[b] < 0) return fail(NVFP4_EINVAL, "n_new[%d] < 0", b);
        if (n_new[b] > 0) {
            if (seq_base[b] < 0 || write_pos[b] < 0 || seq_base[b] + write_pos[b] + n_new[b] > cache->capacity)
                return fail(NVFP4_ERANGE, "sequence %d rows [%lld, %lld) outside the pool", b,
                            (long long)(seq_base[b] + write_pos[b]),
                            (long long)(seq_base[b] + write_pos[b] + n_new[b]));
        }
        p.row_start[b] = acc;
        p.dst_start[b] = seq_base[b] + write_pos[b];
        acc += n_new[b];
    }
    for (int b = num_seqs; b <= nvfp4::kMaxSeqs; ++b) p.row_start[b] = acc;
    if (acc == 0) return ok();
    if (acc * (cache->head_dim / 8) > INT32_MAX)
        return fail(NVFP4_EUNSUPPORTED, "%lld rows in one append call (at most %d for head_dim %d)", (long long)acc,
                    INT32_MAX / (cache->head_dim / 8), cache->head_dim);
    if (!aligned16(k_new) || !aligned16(v_new)) return fail(NVFP4_EINVAL, "k_new/v_new must be non-null and 16-byte aligned");
    p.k_new = static_cast<const uint16_t *>(k_new);
    p.v_new = static_cast<const uint16_t *>(v_new);
    p.gscale = global_scale;
    p.kc = static_cast<uint8_t *>(cache->k_codes);
    p.ks = static_cast<uint8_t *>(cache->k_scales);
    p.vc = static_cast<uint8_t *>(cache->v_codes);
    p.vs = static_cast<uint8_t *>(cache->v_scales);
    p.cap = cache->capacity;
    p.k_fp8 = cache->kv_format == NVFP4_KV_K8V4;
    p.B = num_seqs;
    p.Hkv = cache->num_kv_heads;
    p.D = cache->head_dim;
    p.rows = acc;
    return hip_status(nvfp4::launch_append(p, static_cast<hipStream_t>(stream)), "append launch");
}

size_t nvfp4_decode_attn_workspace_bytes(const nvfp4_kv_cache *cache, int32_t num_seqs, const int64_t *seq_len,
                                         int32_t n_q, int32_t num_q_heads) {
    nvfp4::SplitPlan pl;
    if (make_plan(cache, num_seqs, nullptr, seq_len, n_q, num_q_heads, pl) != NVFP4_OK) return 0;
    return workspace_for(pl);
}

int nvfp4_decode_attn_partial(const nvfp4_kv_cache *cache, const float *global_scale, const void *q,
                              int32_t num_seqs, const int64_t *seq_base, const int64_t *seq_len, int32_t n_q,
                              int32_t num_q_heads, float sm_scale, void *workspace, size_t workspace_bytes,
                              void *stream) {
    nvfp4::SplitPlan pl;
    if (!seq_base) return fail(NVFP4_EINVAL, "seq_base is null");
    int rc = make_plan(cache, num_seqs, seq_base, seq_len, n_q, num_q_heads, pl);
    if (rc) return rc;
    if ((rc = check_decode_common(global_scale, workspace, workspace_bytes, pl))) return rc;
    if (!aligned16(q)) return fail(NVFP4_EINVAL, "q must be non-null and 16-byte aligned");
    if (!std::isfinite(sm_scale)) return fail(NVFP4_EINVAL, "sm_scale must be finite");
    nvfp4::DecodeParams dp;
    fill_decode(dp, pl, cache, global_scale, q, seq_base, seq_len, sm_scale, workspace);
    return hip_status(launch_partials(dp, pl, static_cast<hipStream_t>(stream)), "decode partial launch");
}

int nvfp4_decode_attn_combine(const nvfp4_kv_cache *cache, const float *global_scale, void *out, int32_t out_dtype,
                              int32_t num_seqs, const int64_t *seq_len, int32_t n_q, int32_t num_q_heads,
                              void *workspace, size_t workspace_bytes, void *stream) {
    nvfp4::SplitPlan pl;
    int rc = make_plan(cache, num_seqs, nullptr, seq_len, n_q, num_q_heads, pl);
    if (rc) return rc;
    if ((rc = check_decode_common(global_scale, workspace, workspace_bytes, pl))) return rc;
    if (!aligned16(out)) return fail(NVFP4_EINVAL, "out must be non-null and 16-byte aligned");
    if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_EINVAL, "out_dtype %d invalid", out_dtype);
    nvfp4::DecodeParams dp;
    fill_decode(dp, pl, cache, global_scale, nullptr, nullptr, seq_len, 0.f, workspace);
    dp.out = out;
    dp.out_bf16 = out_dtype == NVFP4_OUT_BF16;
    return hip_status(nvfp4::launch_decode_combine(dp, pl.D, static_cast<hipStream_t>(stream)),
                      "decode combine launch");
}

int nvfp4_decode_step(const nvfp4_kv_cache *cache, const float *global_scale, const void *k_new,
                      const void *v_new, const void *q, void *out, int32_t out_dtype, int32_t num_seqs,
                      const int64_t *seq_base, const int64_t *seq_len, int32_t n_q, int32_t num_q_heads,
                      float sm_scale, void *workspace, size_t workspace_bytes, void *stream) {
    // Validate everything before the first launch so a failed call enqueues nothing.
    nvfp4::SplitPlan pl;
    if (!seq_base) return fail(NVFP4_EINVAL, "seq_base is null");
    int rc = make_plan(cache, num_seqs, seq_base, seq_len, n_q, num_q_heads, pl);
    if (rc) return rc;
    if ((rc = check_decode_common(global_scale, workspace, workspace_bytes, pl))) return rc;
    if (!aligned16(k_new) || !aligned16(v_new))
        return fail(NVFP4_EINVAL, "k_new and v_new must be non-null and 16-byte aligned");
    if (!aligned16(q)) return fail(NVFP4_EINVAL, "q must be non-null and 16-byte aligned");
    if (!aligned16(out)) return fail(NVFP4_EINVAL, "out must be non-null and 16-byte aligned");
    if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_EINVAL, "out_dtype %d invalid", out_dtype);
    if (!std::isfinite(sm_scale)) return fail(NVFP4_EINVAL, "sm_scale must be finite");
    nvfp4::DecodeParams dp;
    fill_decode(dp, pl, cache, global_scale, q, seq_base, seq_len, sm_scale, workspace);
    dp.k_new = static_cast<const uint16_t *>(k_new);
    dp.v_new = static_cast<const uint16_t *>(v_new);
    dp.out = out;
    dp.out_bf16 = out_dtype == NVFP4_OUT_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (pl.R > nvfp4::kMaxStoreRows) {
        // Many row chunks side by side all read the new rows: store them first (append kernel).
        int64_t wp[nvfp4::kMaxSeqs], nn[nvfp4::kMaxSeqs];
        for (int b = 0; b < num_seqs; ++b) {
            wp[b] = seq_len[b] - n_q;
            nn[b] = n_q;
        }
        if ((rc = nvfp4_kv_append(cache, k_new, v_new, global_scale, num_seqs, seq_base, wp, nn, stream)))
            return rc;
    }
    hipError_t e = launch_partials(dp, pl, s);
    if (e != hipSuccess) return hip_status(e, "decode partial launch");
    return hip_status(nvfp4::launch_decode_combine(dp, pl.D, s), "decode combine launch");
}

int nvfp4_decode_step_dev_len(const nvfp4_kv_cache *cache, const float *global_scale, const void *k_new,
                              const void *v_new, const void *q, void *out, int32_t out_dtype, int32_t num_seqs,
                              const int64_t *seq_base, const int64_t *max_len, const int64_t *seq_len_dev,
                              int32_t n_q, int32_t num_q_heads, float sm_scale, void *workspace,
                              size_t workspace_bytes, void *stream) {
    // The plan (grid, units per sequence, workspace) comes from the upper bounds; the
    // kernels split each sequence's units over the length they read from seq_len_dev.
    nvfp4::SplitPlan pl;
    if (!seq_base) return fail(NVFP4_EINVAL, "seq_base is null");
    if (!max_len) return fail(NVFP4_EINVAL, "max_len is null");
    int rc = make_plan(cache, num_seqs, seq_base, max_len, n_q, num_q_heads, pl);
    if (rc) return rc;
    if ((rc = check_decode_common(global_scale, workspace, workspace_bytes, pl))) return rc;
    if (!seq_len_dev || reinterpret_cast<uintptr_t>(seq_len_dev) % 8 != 0)
        return fail(NVFP4_EINVAL, "seq_len_dev must be non-null and 8-byte aligned");
    if ((k_new == nullptr) != (v_new == nullptr))
        return fail(NVFP4_EINVAL, "k_new and v_new must both be given or both be null");
    if (k_new && (!aligned16(k_new) || !aligned16(v_new)))
        return fail(NVFP4_EINVAL, "k_new and v_new must be 16-byte aligned");
    if (k_new && pl.R > nvfp4::kMaxStoreRows)
        return fail(NVFP4_EUNSUPPORTED, "%d query rows per KV head: with lengths in device memory the step "
                    "stores its rows itself only up to 128 rows (append first, pass null k_new/v_new)", pl.R);
    if (!aligned16(q)) return fail(NVFP4_EINVAL, "q must be non-null and 16-byte aligned");
    if (!aligned16(out)) return fail(NVFP4_EINVAL, "out must be non-null and 16-byte aligned");
    if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_EINVAL, "out_dtype %d invalid", out_dtype);
    if (!std::isfinite(sm_scale)) return fail(NVFP4_EINVAL, "sm_scale must be finite");
    nvfp4::DecodeParams dp;
    fill_decode(dp, pl, cache, global_scale, q, seq_base, max_len, sm_scale, workspace);
    dp.len_dev = seq_len_dev;
    dp.k_new = static_cast<const uint16_t *>(k_new);
    dp.v_new = static_cast<const uint16_t *>(v_new);
    dp.out = out;
    dp.out_bf16 = out_dtype == NVFP4_OUT_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_partials(dp, pl, s);
    if (e != hipSuccess) return hip_status(e, "decode partial launch");
    return hip_status(nvfp4::launch_decode_combine(dp, pl.D, s), "decode combine launch");
}

int nvfp4_decode_attn(const nvfp4_kv_cache *cache, const float *global_scale, const void *q, void *out,
                      int32_t out_dtype, int32_t num_seqs, const int64_t *seq_base, const int64_t *seq_len,
                      int32_t n_q, int32_t num_q_heads, float sm_scale, void *workspace, size_t workspace_bytes,
                      void *stream) {
    // Validate everything before the first launch so a failed call enqueues nothing.
    nvfp4::SplitPlan pl;
    if (!seq_base) return fail(NVFP4_EINVAL, "seq_base is null");
    int rc = make_plan(cache, num_seqs, seq_base, seq_len, n_q, num_q_heads, pl);
    if (rc) return rc;
    if ((rc = check_decode_common(global_scale, workspace, workspace_bytes, pl))) return rc;
    if (!aligned16(q)) return fail(NVFP4_EINVAL, "q must be non-null and 16-byte aligned");
    if (!aligned16(out)) return fail(NVFP4_EINVAL, "out must be non-null and 16-byte aligned");
    if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16)
        return fail(NVFP4_EINVAL, "out_dtype %d invalid", out_dtype);
    if (!std::isfinite(sm_scale)) return fail(NVFP4_EINVAL, "sm_scale must be finite");
    nvfp4::DecodeParams dp;
    fill_decode(dp, pl, cache, global_scale, q, seq_base, seq_len, sm_scale, workspace);
    dp.out = out;
    dp.out_bf16 = out_dtype == NVFP4_OUT_BF16;
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = launch_partials(dp, pl, s);
    if (e != hipSuccess) return hip_status(e, "decode partial launch");
    return hip_status(nvfp4::launch_decode_combine(dp, pl.D, s), "decode combine launch");
}

int nvfp4_hbm_read_probe(const void *buf, size_t bytes, void *sink, int32_t workgroups, void *stream) {
    if (!aligned16(buf)) return fail(NVFP4_EINVAL, "buf must be non-null and 16-byte aligned");
    if (bytes < 16 || bytes % 16 != 0) return fail(NVFP4_EINVAL, "bytes must be a positive multiple of 16");
    if (!sink || reinterpret_cast<uintptr_t>(sink) % 4 != 0)
        return fail(NVFP4_EINVAL, "sink must be non-null and 4-byte aligned");
    if (workgroups < 1 || workgroups > 65536) return fail(NVFP4_EINVAL, "workgroups must be in [1, 65536]");
    return hip_status(nvfp4::launch_read_probe(buf, bytes, static_cast<uint32_t *>(sink), workgroups,
                                               static_cast<hipStream_t>(stream)),
                      "read probe launch");
}

}  // extern "C"
