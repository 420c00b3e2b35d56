// Internal declarations shared by the host API and the kernel launchers.
// Nothing here is part of the public ABI (include/nvfp4_kv.h is).
#pragma once

#include <stdint.h>
#include <hip/hip_runtime.h>

namespace nvfp4 {

constexpr int kMaxSeqs = 8;
constexpr int kMaxRows = 64;       // query rows per KV head one decode launch serves per chunk
constexpr int kChunkRows = 32;     // above kMaxRows: row chunks of this size side by side
constexpr int kMaxStoreRows = 128; // up to this many rows the decode kernels store a step's rows
constexpr int kBlockTokens = 32;     // tokens per KV block: one PV MFMA K-step (16x16x32)
constexpr int kWaves = 4;            // waves per decode workgroup (256 threads)
constexpr int kCUs = 256;            // compute units the split plan fills (MI355X)
// Longest unit the split planner makes. Probabilities enter the PV product in fp16 against
// the running reference of one wave (or wave pair); a weight below 2^-25 of that reference
// rounds to 0 (below 2^-14 it keeps only absolute precision 2^-25). A wave sees at most a
// quarter of a unit, so this caps the mass lost to that floor at 8192 x 2^-24 (about 4.9e-4)
// of the output's V range, next to the 2^-10 bound of fp16 rounding in the normal range.
constexpr int kMaxUnitTokens = 32768;

// Waves per SIMD that the partial kernel for NT row tiles is built for, set by its register
// budget: two everywhere (one or two row tiles: the single-wave-per-block kernel, up to 256
// VGPRs; three or four: the pair kernel, one 8-wave workgroup per CU).
constexpr int decode_waves_per_simd(int /*NT*/) { return 2; }
// Wave pairs per workgroup of the pair kernel (three or four row tiles): one workgroup holds
// every pair a CU keeps resident (8 waves); with several workgroups per CU the
// later-dispatched ones ran slower and set the kernel's end, and one workgroup halves the
// partials (mtp_verify step 58.9 -> 56.5 us).
constexpr int decode_pairs_per_wg(int /*NT*/) { return 4; }
// Units the split planner gives each CU: one. One row tile: a 4-wave workgroup, although
// two such workgroups fit -- half as many, twice as long units pay the per-unit start and
// merge half as often (decode at 2 x 32k tokens: partial 21.6 -> 20.2 us; 600k: 123.1 ->
// 121.7 us). Two row tiles: one 8-wave workgroup (two waves per SIMD) whose waves claim the
// unit's blocks one at a time; as two 4-wave workgroups with static blocks, the one
// dispatched second ran ~40% slower and finished alone (three sessions of 330k-470k tokens,
// 24 rows: step 259.4 -> 254.4 us). Three or four: one 8-wave pair-kernel workgroup.
constexpr int decode_units_per_cu(int /*NT*/) { return 1; }
// Waves per workgroup of the one-wave-per-block kernel (one or two row tiles).
constexpr int decode_partial_waves(int NT) { return NT == 2 ? 8 : 4; }

// Split-K plan: sequence b is cut into n_split[b] units of split_len[b] tokens
// (a multiple of kBlockTokens) for each KV head; the last unit ends at the
// sequence length and holds at least n_q tokens (so the rows a decode step
// appends all fall in it). Units are numbered sequence-major, then KV head, then
// split.
struct SplitPlan {
    int32_t B, Hkv, Hq, G, n_q, R, NT, D;
    int32_t chunk_rows;                  // rows per row chunk (the last may have fewer)
    int32_t chunks;                      // row chunks, side by side on grid y (1: R <= 64)
    int32_t n_split[kMaxSeqs];
    int32_t split_len[kMaxSeqs];
    int32_t unit_base[kMaxSeqs];
    int32_t units;
};

// Kernel parameters of the decode pair (passed by value).
struct DecodeParams {
    uint8_t *kc, *ks, *vc, *vs;          // pool planes (written only by the step's own append)
    int64_t cap;
    int32_t k_fp8;                       // K planes: 0 NVFP4; 1 row-scaled FP8 E4M3 (K8V4)
    const float *gscale;                 // [B][Hkv][2]
    const uint16_t *q;                   // bf16 [B][n_q][Hq][D]
    const uint16_t *k_new, *v_new;       // bf16 [B n_q][Hkv][D] rows to append first, or null
    const int64_t *len_dev;              // device lengths [B] read at run time, or null (then
                                         // seq_len holds the lengths; else their upper bounds)
    float *ws_o, *ws_m, *ws_l;           // [units][R][D], [units][R], [units][R]
    void *out;
    int32_t out_bf16;
    float sm_scale;
    int32_t B, Hkv, Hq, G, n_q, R;       // R = G n_q rows per KV head (workspace stride)
    int32_t row0, Rc;                    // rows of the workgroups with blockIdx.y = y:
                                         // [row0 + y Rc, min(row0 + (y + 1) Rc, R)), Rc <= 64
    int32_t grid_y;                      // row chunks run side by side (grid y), >= 1
    int64_t seq_base[kMaxSeqs];
    int64_t seq_len[kMaxSeqs];
    int32_t n_split[kMaxSeqs];
    int32_t split_len[kMaxSeqs];
    int32_t unit_base[kMaxSeqs];
    int32_t units;
};

struct AppendParams {
    const uint16_t *k_new, *v_new;       // bf16 [rows][Hkv][D]
    const float *gscale;                 // [B][Hkv][2]
    uint8_t *kc, *ks, *vc, *vs;
    int64_t cap;
    int32_t k_fp8;                       // K planes: 0 NVFP4; 1 row-scaled FP8 E4M3 (K8V4)
    int32_t B, Hkv, D;
    int64_t rows;                        // sum of n_new
    int64_t row_start[kMaxSeqs + 1];     // prefix sums of n_new
    int64_t dst_start[kMaxSeqs];         // seq_base + write_pos
};

struct CalibParams {
    const uint16_t *k_rows, *v_rows;     // bf16 [rows][Hkv][D]
    float *gscale;                       // [B][Hkv][2]
    int32_t B, Hkv, D;
    int64_t row_start[kMaxSeqs + 1];
};

// Records the thread's last error message (nvfp4_last_error) and returns code.
int report_error(int code, const char *fmt, ...);

hipError_t launch_calibrate(const CalibParams &p, hipStream_t s);
hipError_t launch_append(const AppendParams &p, hipStream_t s);
// NT 1..2: the four waves take alternate blocks; NT 3..4: the wave-pair kernel.
hipError_t launch_decode_partial(const DecodeParams &p, int D, int NT, hipStream_t s);
hipError_t launch_decode_pair(const DecodeParams &p, int D, int NT, hipStream_t s);
hipError_t launch_decode_combine(const DecodeParams &p, int D, hipStream_t s);
hipError_t launch_read_probe(const void *buf, uint64_t bytes, uint32_t *sink, int workgroups, hipStream_t s);

}  // namespace nvfp4
