/*
 * nvfp4_kv.h -- C ABI of the MI355X (gfx950) NVFP4-KV decode-attention library.
 *
 * The method (gzenz/ninfer page, section "Context and model", bullet "NVFP4 KV
 * cache"): K and V rows are stored as 4-bit E2M1 codes with one E4M3 scale per
 * group of 16 elements, "45% less KV VRAM than int8". The calls follow the
 * pages' statement of the problem: a per-engine KV dtype, one startup-fixed KV
 * pool shared by the active requests, each request with its own logical length
 * (knoopx/ninfer page, "Capabilities and limits": one to eight active requests,
 * "one shared startup-fixed KV pool", MTP draft windows of one to five, format
 * and shape combinations served by explicitly implemented native paths, so
 * unsupported ones are rejected, not emulated).
 *
 * ---------------------------------------------------------------- layout ----
 * A pool holds, for each of num_kv_heads heads and capacity token slots:
 *   k_codes, v_codes   uint8 [num_kv_heads][capacity][head_dim/2]
 *                      byte j of a row = code(2j) | code(2j+1) << 4 (even element
 *                      in the low nibble); a code is sign<<3 | E2M1 magnitude code.
 *   k_scales, v_scales uint8 [num_kv_heads][capacity][head_dim/16]
 *                      byte j = E4M3 (OCP E4M3FN) code of the scale of elements
 *                      [16j, 16j+16); always in 0x00..0x7E (never negative/NaN).
 *   global_scale       float [num_seqs][num_kv_heads][2], index 0 = K, 1 = V:
 *                      g = fp32(amax / (6*448)) over that sequence's rows of that
 *                      head (second-level scale; not on the pages, a stated reading).
 * Element value: x_hat = e2m1(code) * e4m3(scale) * g.
 * K8V4 pools (kv_format = NVFP4_KV_K8V4: 8-bit K with 4-bit V, knoopx/ninfer page,
 * "Capabilities and limits", KV storage list) keep V as above and store K row-scaled in
 * FP8 E4M3, the engine's 8-bit KV format (knoopx/ninfer page, "Performance": FP8 E4M3
 * row-256; the pages do not say which 8-bit format K8V4's K uses, so this is a reading):
 *   k_codes   uint8 [num_kv_heads][capacity][head_dim], byte d = E4M3FN code of element d
 *             (sign << 7 | magnitude code 0x00..0x7E)
 *   k_scales  float [num_kv_heads][capacity], the row scale s = fp32(amax_row / 448)
 *   K element value: e4m3(code) * s; global_scale[b][h][0] is not used for K.
 *   Bytes per (token, KV head): head_dim + 4 for K, head_dim/2 + head_dim/16 for V.
 * Sequence b owns slots [seq_base[b], seq_base[b] + length) in every head plane.
 * Quantisation rounds the exact real ratios amax_group/(6g) and |x|/(S g) to the
 * nearest E4M3 / E2M1 value, ties to the even code, saturating at 448 / 6; the
 * input's sign bit becomes the code's sign bit; g == 0 gives scale 0 and zero
 * magnitudes. K8V4's K rows: each element's code is the E4M3 value nearest the exact real
 * |x| / s, ties to the even code, saturating at 448, sign bit copied; s == 0 gives zero
 * magnitudes.
 *
 * ------------------------------------------------------------ conventions ---
 * - Every device pointer is allocated and owned by the caller. The library never
 *   allocates, frees or synchronises; each call validates its arguments on the
 *   host, then only enqueues kernels on `stream` (a hipStream_t; NULL = the
 *   default stream) and returns. Host arrays are read during the call only.
 * - Device pointers must be 16-byte aligned. bf16 is IEEE bfloat16 bit patterns.
 * - Functions are stateless and thread-safe; the last error message is
 *   thread-local.
 * - Return value: 0 on success, else one of the negative codes below, checked
 *   before any launch (a failed call enqueues nothing), except NVFP4_EHIP which
 *   reports a launch failure. NaN or infinite inputs in device memory are the
 *   caller's responsibility (results are then unspecified).
 */
#ifndef NVFP4_KV_H
#define NVFP4_KV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_OK            0
#define NVFP4_EINVAL       (-1)  /* null or unaligned pointer, count out of range      */
#define NVFP4_EUNSUPPORTED (-2)  /* shape with no native path (see each call)           */
#define NVFP4_ERANGE       (-3)  /* slots past capacity, length shorter than n_q        */
#define NVFP4_EWORKSPACE   (-4)  /* workspace smaller than the size query returned      */
#define NVFP4_EHIP         (-5)  /* a kernel launch failed (message: nvfp4_last_error)  */

#define NVFP4_OUT_F32  0
#define NVFP4_OUT_BF16 1

#define NVFP4_KV_NVFP4 0         /* kv_format: K and V both NVFP4                      */
#define NVFP4_KV_K8V4  1         /* kv_format: row-scaled FP8 E4M3 K, NVFP4 V          */

#define NVFP4_MAX_SEQS 8         /* active sequences per call                         */
#define NVFP4_MAX_ROWS 8192      /* GQA group x query tokens sharing one KV head      */

/* The caller-owned pool. head_dim must be 128 or 256; num_kv_heads >= 1;
 * capacity >= 1 token slots per head plane, and one head's largest code plane in bytes
 * (capacity * head_dim / 2; capacity * head_dim for K8V4's K) at most 2^31 - 1, since
 * kernels address a head plane with 32-bit offsets (else NVFP4_EUNSUPPORTED).
 * kv_format: NVFP4_KV_NVFP4 or NVFP4_KV_K8V4 (else NVFP4_EINVAL). */
typedef struct nvfp4_kv_cache {
    void   *k_codes;
    void   *k_scales;
    void   *v_codes;
    void   *v_scales;
    int32_t num_kv_heads;
    int32_t head_dim;
    int64_t capacity;
    int32_t kv_format;
} nvfp4_kv_cache;

/* Global scales from the rows that will be stored (second-level per-(sequence,
 * KV head) scale; a stated reading, the pages do not give it).
 *   k_rows, v_rows: device bf16 [sum(n_rows)][num_kv_heads][head_dim], the rows of
 *                   sequence 0, then sequence 1, ...
 *   n_rows:         host int64 [num_seqs], each >= 0 (0 gives g = 0)
 *   global_scale:   device float [num_seqs][num_kv_heads][2], written:
 *                   g[b][h][0|1] = fp32(max |x| over sequence b's K|V rows of head h / 2688)
 * Errors: EINVAL (null/unaligned pointers, num_seqs < 1, n_rows < 0),
 *         EUNSUPPORTED (num_seqs > 8, head_dim not 128/256). */
int nvfp4_kv_calibrate(const nvfp4_kv_cache *cache, const void *k_rows, const void *v_rows,
                       int32_t num_seqs, const int64_t *n_rows, float *global_scale,
                       void *stream);

/* Quantise-on-append (gzenz/ninfer page, "Context and model", NVFP4 KV cache bullet: K
 * and V kept as E2M1 codes with E4M3 group-16 scales; knoopx/ninfer page, "Capabilities and
 * limits": each request's rows go into the one shared, startup-fixed KV pool at its own
 * slots): writes n_new[b] K and V rows of sequence b at slots
 * seq_base[b] + write_pos[b] + r (r < n_new[b]) of every head plane. Lengths are
 * the caller's to advance. Each 16-element group gets its E4M3 scale from its own
 * maximum and the given g; rows whose values exceed 2688 g saturate.
 *   k_new, v_new:  device bf16 [sum(n_new)][num_kv_heads][head_dim], concatenated over b
 *   global_scale:  device float [num_seqs][num_kv_heads][2]
 *   seq_base, write_pos, n_new: host int64 [num_seqs]; n_new[b] >= 0
 * Errors: EINVAL, EUNSUPPORTED (num_seqs > 8, head_dim, sum(n_new) * head_dim / 8
 *         above 2^31 - 1), ERANGE (a slot outside [0, capacity)). Sequences must not
 *         write overlapping slots. */
int nvfp4_kv_append(const nvfp4_kv_cache *cache, const void *k_new, const void *v_new,
                    const float *global_scale, int32_t num_seqs, const int64_t *seq_base,
                    const int64_t *write_pos, const int64_t *n_new, void *stream);

/* Bytes of device workspace nvfp4_decode_attn (and its two halves below) need
 * for these arguments; 0 if the arguments are invalid (the decode call then
 * reports why). The split-K plan depends only on the arguments. The caller owns and
 * allocates the workspace, as it owns the pool (knoopx/ninfer page, "Capabilities and
 * limits": the shared KV pool is sized at startup and stays fixed for the process lifetime,
 * so a caller sizes this buffer once for its largest step). */
size_t nvfp4_decode_attn_workspace_bytes(const nvfp4_kv_cache *cache, int32_t num_seqs,
                                         const int64_t *seq_len, int32_t n_q,
                                         int32_t num_q_heads);

/* Grouped-query decode attention read directly from the NVFP4 pool (gzenz/ninfer page,
 * "Context and model": attention over the NVFP4 KV cache; knoopx/ninfer page, "Capabilities
 * and limits": one to eight active requests decoded as one batch, each with 1 + 1..5 MTP
 * draft tokens verified together, hence n_q query tokens causal among themselves).
 *   q:        device bf16 [num_seqs][n_q][num_q_heads][head_dim]
 *   out:      device [num_seqs][n_q][num_q_heads][head_dim], fp32 or bf16 (out_dtype;
 *             bf16 is the round-to-nearest-even of the fp32 result)
 *   seq_len:  host int64 [num_seqs]; the length INCLUDES the n_q query tokens, whose
 *             K/V rows were already appended. Query token i of sequence b sees keys
 *             [0, seq_len[b] - n_q + i] (bottom-right causal among the n_q tokens).
 *   seq_base: host int64 [num_seqs]
 *   Query head h reads KV head h / (num_q_heads / num_kv_heads).
 *   out = softmax(sm_scale * q . k_hat) . v_hat, computed with fp32 accumulation.
 *   Up to 64 query rows per KV head ((num_q_heads/num_kv_heads) * n_q) are served by one
 *   pass over the cache; 65..8192 rows (wide draft windows, e.g. n_q = 16 at a GQA group
 *   of 6, and prefill chunks attending to the cache and, causally, to themselves) by
 *   32-row chunks side by side in one launch, each chunk reading the KV blocks its rows
 *   can see (chunks of one unit run at the same time, so most repeated reads hit cache).
 * Errors: EINVAL (pointers, out_dtype, n_q < 1, non-finite sm_scale),
 *         EUNSUPPORTED (head_dim, num_q_heads % num_kv_heads != 0, num_seqs > 8,
 *         (num_q_heads/num_kv_heads) * n_q > 8192), ERANGE (seq_len < n_q, slots past
 *         capacity), EWORKSPACE (workspace_bytes below the size query). */
int nvfp4_decode_attn(const nvfp4_kv_cache *cache, const float *global_scale, const void *q,
                      void *out, int32_t out_dtype, int32_t num_seqs, const int64_t *seq_base,
                      const int64_t *seq_len, int32_t n_q, int32_t num_q_heads, float sm_scale,
                      void *workspace, size_t workspace_bytes, void *stream);

/* One decode step of the batch (knoopx/ninfer page, "Capabilities and limits": batched
 * decode of one to eight requests and MTP verification of one to five drafts, run as
 * exact-batch graphs): stores the step's n_q new K/V rows of every sequence, then
 * attends over the whole sequence. Equivalent to
 *   nvfp4_kv_append(cache, k_new, v_new, global_scale, num_seqs, seq_base,
 *                   write_pos = seq_len - n_q, n_new = n_q, stream)
 * followed by nvfp4_decode_attn(...) with the same arguments, and bit-identical to
 * that pair (pool bytes and out); the rows are quantised inside the decode kernel by
 * the workgroups that read them, so the step is two kernel launches instead of three.
 *   k_new, v_new: device bf16 [num_seqs * n_q][num_kv_heads][head_dim], sequence 0's
 *                 n_q rows first; row r of sequence b goes to slot
 *                 seq_base[b] + seq_len[b] - n_q + r. (Above 128 query rows per KV head
 *                 -- a prefill chunk -- the rows are stored by the append kernel first:
 *                 three launches.)
 *   Other arguments, the workspace and the errors as for nvfp4_decode_attn (EINVAL
 *   also for null or unaligned k_new / v_new). */
int nvfp4_decode_step(const nvfp4_kv_cache *cache, const float *global_scale, const void *k_new,
                      const void *v_new, const void *q, void *out, int32_t out_dtype,
                      int32_t num_seqs, const int64_t *seq_base, const int64_t *seq_len,
                      int32_t n_q, int32_t num_q_heads, float sm_scale, void *workspace,
                      size_t workspace_bytes, void *stream);

/* The decode step with the lengths in device memory (knoopx/ninfer page, "Capabilities and
 * limits": decode replayed as exact-batch graphs). The kernels read seq_len_dev when they
 * run, so a HIP graph that captured this call replays across decode steps while the
 * sequences grow: the caller updates seq_len_dev (and the contents of q, k_new, v_new)
 * between replays. The launch configuration is fixed by max_len: the split planner runs on
 * max_len on the host; each kernel divides a sequence's fixed number of units over the
 * length it reads (units past it are empty). Per replay, the result equals
 * nvfp4_decode_step with seq_len = the device values (same pool bytes; out within the
 * attention tolerance, the split points may differ).
 *   max_len:     host int64 [num_seqs], an upper bound on every seq_len_dev[b] the graph
 *                will see; validated as seq_len is for nvfp4_decode_step (n_q <= max_len,
 *                seq_base + max_len within capacity); it sizes the workspace:
 *                nvfp4_decode_attn_workspace_bytes(cache, num_seqs, max_len, n_q, num_q_heads)
 *   seq_len_dev: device int64 [num_seqs], 8-byte aligned; read at run time. A value outside
 *                [n_q, max_len[b]] is a caller error: the kernels clamp it into that range
 *                (no access outside the sequence's slots; the result is then meaningless).
 *   k_new, v_new: as for nvfp4_decode_step, or both null: attention only, no append.
 *   Other arguments, the workspace and the errors as for nvfp4_decode_step (EINVAL also
 *   for a null or unaligned seq_len_dev, or only one of k_new / v_new null; EUNSUPPORTED
 *   for k_new with more than 128 query rows per KV head: append those rows first). */
int nvfp4_decode_step_dev_len(const nvfp4_kv_cache *cache, const float *global_scale, const void *k_new,
                              const void *v_new, const void *q, void *out, int32_t out_dtype,
                              int32_t num_seqs, const int64_t *seq_base, const int64_t *max_len,
                              const int64_t *seq_len_dev, int32_t n_q, int32_t num_q_heads,
                              float sm_scale, void *workspace, size_t workspace_bytes, void *stream);

/* Capacity of the static scratch array that nvfp4_decode_step_noalloc uses (MiB). */
#define NVFP4_NOALLOC_SCRATCH_MIB 32

/* nvfp4_decode_step for callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation. Same arguments, results
 * and errors as nvfp4_decode_step, without the workspace: the split-K partials go to a
 * fixed device array inside the library (NVFP4_NOALLOC_SCRATCH_MIB MiB per GPU, held until
 * the process ends). The call allocates nothing; its first call on a device looks the
 * array's address up (hipGetSymbolAddress).
 *   - A step whose partials need more than the array holds (the size query
 *     nvfp4_decode_attn_workspace_bytes says how many bytes) is rejected with
 *     NVFP4_EWORKSPACE before any launch; nvfp4_decode_step with a caller workspace serves it.
 *   - Every call on one GPU shares that GPU's array: calls that may overlap in time (on
 *     different streams) race and give wrong results. Calls on one stream are ordered.
 *   - NVFP4_EHIP also if the device or the array's address cannot be queried. */
int nvfp4_decode_step_noalloc(const nvfp4_kv_cache *cache, const float *global_scale, const void *k_new,
                              const void *v_new, const void *q, void *out, int32_t out_dtype,
                              int32_t num_seqs, const int64_t *seq_base, const int64_t *seq_len,
                              int32_t n_q, int32_t num_q_heads, float sm_scale, void *stream);

/* The two kernels of nvfp4_decode_attn (the same attention as nvfp4_decode_attn, whose
 * passages they follow), callable on their own (same arguments, same workspace) so that each
 * can be timed: the split-K partial pass writes per-split (o, m, l) into the workspace; the
 * combine pass merges them by log-sum-exp, applies the V global scale and writes out. */
int nvfp4_decode_attn_partial(const nvfp4_kv_cache *cache, const float *global_scale,
                              const void *q, int32_t num_seqs, const int64_t *seq_base,
                              const int64_t *seq_len, int32_t n_q, int32_t num_q_heads,
                              float sm_scale, void *workspace, size_t workspace_bytes,
                              void *stream);
int nvfp4_decode_attn_combine(const nvfp4_kv_cache *cache, const float *global_scale,
                              void *out, int32_t out_dtype, int32_t num_seqs,
                              const int64_t *seq_len, int32_t n_q, int32_t num_q_heads,
                              void *workspace, size_t workspace_bytes, void *stream);

/* Streaming-read probe (measurement only, not part of the decode path): reads `bytes` of
 * device memory at `buf` once with 16-byte non-temporal loads (the policy of the decode
 * kernels' KV loads) from `workgroups` 256-thread workgroups and
 * writes one fold of the data per workgroup to sink[0 .. workgroups). Timing it gives the
 * read rate a plain streaming kernel reaches, the practical ceiling for the decode kernels
 * (knoopx/ninfer page, "Quick start": the engine ships a standalone HBM probe).
 *   buf:  device, 16-byte aligned; bytes a positive multiple of 16
 *   sink: device uint32 [workgroups], 4-byte aligned; contents are a checksum, not a result
 * Errors: EINVAL (pointers, bytes, workgroups outside [1, 65536]). */
int nvfp4_hbm_read_probe(const void *buf, size_t bytes, void *sink, int32_t workgroups, void *stream);

/* Message describing the last failure on this thread ("" if none). */
const char *nvfp4_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_KV_H */
