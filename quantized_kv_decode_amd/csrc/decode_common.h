// Device helpers shared by the decode kernels (fp4/fp16 packing, buffer
// resources, the query prologue and the split-unit lookup).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "internal.h"
#include "quantize.h"

namespace nvfp4 {
namespace dev {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLazyMax = 8.0f;      // raise the softmax reference only past m + 8 (base 2)
// Smallest score factor (see q_store). NVFP4 K: MFMA scores are below 2^27 in magnitude
// (|q| < 2^15 per element after scaling, |k_hat'| <= 6 * 448 * 2^-8 = 10.5, 256 terms), so a
// score times this is below 2^-72. FP8 K (K8V4): scores are below 2^32 times the key's row
// scale (amax_row / 448), so below 2^-67 times amax_row: negligible unless K's magnitudes
// exceed about 10^15.
constexpr float kMinScoreScale = 1e-30f;

__device__ inline half2_t as_h2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }
__device__ inline uint32_t as_u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// fp16 pair (S * 2^-8, S * 2^-8) from an E4M3 byte 0x00..0x7E.
__device__ inline uint32_t scale_pair(uint32_t byte) { return (byte << 7) | (byte << 23); }

template <int SEL>
__device__ inline uint32_t fp4x2(uint32_t w) {
    return as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL));
}

__device__ inline uint32_t hmul2(uint32_t a, uint32_t b) { return as_u32(as_h2(a) * as_h2(b)); }

__device__ inline uint32_t bfi(uint32_t mask, uint32_t a, uint32_t b) { return (a & mask) | (b & ~mask); }

// max over the four lane groups (lanes n, n+16, n+32, n+48), on the VALU: permlane16_swap of
// x with itself yields rows (0,0,2,2) and (1,1,3,3); permlane32_swap of y with itself yields
// halves (lo,lo) and (hi,hi).
__device__ inline float wave_max_g(float x) {
    const uint32_t xb = __builtin_bit_cast(uint32_t, x);
    const auto a = __builtin_amdgcn_permlane16_swap(xb, xb, false, false);
    const float y = fmaxf(__builtin_bit_cast(float, (uint32_t)a[0]), __builtin_bit_cast(float, (uint32_t)a[1]));
    const uint32_t yb = __builtin_bit_cast(uint32_t, y);
    const auto c = __builtin_amdgcn_permlane32_swap(yb, yb, false, false);
    return fmaxf(__builtin_bit_cast(float, (uint32_t)c[0]), __builtin_bit_cast(float, (uint32_t)c[1]));
}

// Maximum of 8 scores in four VALU instructions. Written out because fmaxf on values the
// compiler cannot prove quiet (MFMA results, masked -inf) gets a quieting v_max x, x per
// operand first; scores are never NaN.
__device__ inline float max8(const float (&x)[8]) {
    float a, b, c, r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(a) : "v"(x[0]), "v"(x[1]), "v"(x[2]));
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(b) : "v"(x[3]), "v"(x[4]), "v"(x[5]));
    asm("v_max_f32 %0, %1, %2" : "=v"(c) : "v"(x[6]), "v"(x[7]));
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

__device__ inline float max4(const float (&x)[4]) {
    float a, r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(a) : "v"(x[0]), "v"(x[1]), "v"(x[2]));
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(x[3]));
    return r;
}

typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Cache policy of the KV plane loads. Code loads (whole lines, every byte read once per
// step) use nt, the non-temporal streaming policy: a plain 16-byte read sweep of 1 GiB on
// MI355X went from 6.38 to 7.07 TB/s with it. Scale loads (a few bytes per lane, several
// lanes per line) keep the default policy: same box, A/B in one process, per decode step,
// streaming codes with default-policy scales against streaming everything: 237.9 vs 249.1 us
// (three sessions of 330k-470k tokens), 106.1 vs 114.8 us (600k tokens), 49.8 vs 51.3 us
// (MTP verify, 131k). The FP8 K codes of K8V4 keep the default policy too (with streaming
// K loads that decode took 443 us per step, without 327 us).
constexpr int kCodePolicy = 2;           // nt
constexpr int kScalePolicy = 0;
template <int KF>
constexpr int kKCodePolicy = KF ? 0 : kCodePolicy;

// Raw buffer over one head plane: loads past its end return zeros (no fault).
__device__ inline rsrc_t plane_rsrc(const uint8_t *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t *>(base), (short)0, (int)bytes, 0x00020000);
}

// Byte offsets of one lane's first load in each stream for the block starting at
// slot `slot0` (= seq_base + block start); later tokens of the block are
// immediate offsets. Tokens past the sequence end are read (finite values, or
// zeros past the plane) and masked out of the softmax.
struct Offs {
    uint32_t kc, ks, vc, vs;
};

// Geometry of the K planes: KF = 0, NVFP4 (D/2 code bytes and D/16 E4M3 scale bytes per
// token row); KF = 1, row-scaled FP8 E4M3 of K8V4 (D code bytes and one fp32 scale per row).
// V planes are NVFP4 either way.
template <int D, int KF>
struct KGeom {
    static constexpr int CB = KF ? D : D / 2;          // K code bytes per token row
    static constexpr int SB = KF ? 4 : D / 16;         // K scale bytes per token row
};

// Byte offsets of a block starting at token slot slot0: lane part + slot part (32-bit:
// a head plane is below 2^31 bytes).
template <int D, int KF>
__device__ inline Offs add_slot(const Offs &lane, uint32_t slot0) {
    Offs o;
    o.kc = lane.kc + slot0 * (uint32_t)KGeom<D, KF>::CB;
    o.ks = lane.ks + slot0 * (uint32_t)KGeom<D, KF>::SB;
    o.vc = lane.vc + slot0 * (uint32_t)(D / 2);
    o.vs = lane.vs + slot0 * (uint32_t)(D / 16);
    return o;
}

// fp16 pair of the two E4M3 bytes in the low (SEL = 0) or high (SEL = 1) half of w: exact
// (every E4M3 value is an fp16 value; the scale operand 1.0 leaves them unchanged).
template <int SEL>
__device__ inline uint32_t fp8x2(uint32_t w) {
    return as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, SEL != 0));
}

// Head planes are below 2^31 bytes (the capacity limit), so this offset, plus any
// immediate offset of a block's loads, is out of range for every plane.
constexpr uint32_t kPastPlane = 0x80000000u;

// Unit u of the split plan: sequence b, KV head kh, tokens [t0, t1) of the
// sequence (length L), nblk 32-token blocks; last: the unit ending at L.
struct Unit {
    int b, kh, nblk;
    bool last;
    int64_t L, t0, t1;
};

// DevLen: the lengths are read from p.len_dev when the kernel runs (a separate kernel
// instantiation, so that the host-length kernels carry none of its code).
template <bool DevLen>
__device__ inline Unit unit_of(const DecodeParams &p, int u) {
    Unit r;
    r.b = 0;
#pragma unroll
    for (int s = 1; s < kMaxSeqs; ++s)
        if (s < p.B && u >= p.unit_base[s]) r.b = s;
    const int local = u - p.unit_base[r.b];
    const int ns = p.n_split[r.b];
    r.kh = local / ns;
    const int sp = local - r.kh * ns;
    if constexpr (!DevLen) {
        r.L = p.seq_len[r.b];
        r.last = sp == ns - 1;
        r.t0 = (int64_t)sp * p.split_len[r.b];
        r.t1 = r.last ? r.L : r.t0 + p.split_len[r.b];
    } else {
        // Lengths read when the kernel runs (a captured graph replays across steps): the
        // same split rule as the host planner, over the sequence's fixed number of units;
        // units past the length are empty. Out-of-range lengths are clamped into
        // [n_q, upper bound], so no access leaves the sequence's slots.
        // readfirstlane: the loaded length is the same in every lane; without it the unit's
        // range (and the block loop's control on both paths) would live in vector registers
        const int Ld = __builtin_amdgcn_readfirstlane((int)min(max(p.len_dev[r.b], (int64_t)p.n_q), p.seq_len[r.b]));
        const int L = Ld;
        int sl = (L + ns - 1) / ns;
        // At least n_q tokens per unit: with a short length over many planned units the
        // step's n_q new rows would otherwise reach into the unit before the last one, whose
        // workgroup would read slots that the last unit's workgroup is storing.
        sl = max(sl, p.n_q);
        sl = (sl + kBlockTokens - 1) / kBlockTokens * kBlockTokens;
        int ne = (L + sl - 1) / sl;
        if (ne > 1 && L - (ne - 1) * sl < p.n_q) ne -= 1;    // the newest n_q tokens stay in one unit
        r.L = L;
        r.last = sp == ne - 1;
        r.t0 = sp < ne ? (int64_t)sp * sl : (int64_t)L;
        r.t1 = sp < ne ? (r.last ? (int64_t)L : r.t0 + sl) : (int64_t)L;
    }
    r.nblk = (int)((r.t1 - r.t0 + kBlockTokens - 1) / kBlockTokens);
    return r;
}

// The query rows of this workgroup: [row0, row0 + Rc) of the KV head's R = G n_q rows
// (row = query token x G + head in the group). Row chunks launched side by side take the
// chunk index from blockIdx.y.
struct Rows {
    int row0, Rc;
};

__device__ inline Rows rows_of(const DecodeParams &p) {
    const int row0 = p.row0 + (int)blockIdx.y * p.Rc;
    return Rows{row0, min(p.Rc, p.R - row0)};
}

// Causal trim: keys past the last one that the workgroup's last query token sees are
// masked for all its rows, so the unit's range stops there (whole blocks are skipped; the
// result is unchanged). Matters for long query chunks (prefill).
__device__ inline void trim_causal(Unit &un, const DecodeParams &p, const Rows &rw) {
    const int64_t i_last = (rw.row0 + rw.Rc - 1) / p.G;
    const int64_t kend = un.L - p.n_q + i_last + 1;
    if (un.t1 > kend) {
        un.t1 = kend > un.t0 ? kend : un.t0;
        un.nblk = (int)((un.t1 - un.t0 + kBlockTokens - 1) / kBlockTokens);
    }
}

// One 16-element group of a K row of a K8V4 pool: the row's scale from the maxima of its
// D/16 groups, held by D/16 consecutive lanes aligned to D/16 (all active together), then
// the group's 16 code bytes; the row's first lane also stores the scale.
template <int D>
__device__ inline void store_fp8_group(const uint32_t (&w)[8], int j, uint8_t *kc, uint8_t *ks, int64_t plane_row) {
    uint32_t am = amax16_bits(w);
#pragma unroll
    for (int off = 1; off < D / 16; off <<= 1) am = max(am, (uint32_t)__shfl_xor((int)am, off));
    const float s = fp8_row_scale(am);
    uint32_t c[4];
    fp8_row_codes(w, s, c);
    *reinterpret_cast<uint4 *>(kc + plane_row * D + 16 * j) = make_uint4(c[0], c[1], c[2], c[3]);
    if (j == 0) reinterpret_cast<float *>(ks)[plane_row] = s;
}

// The n_q rows a decode step appends for (sequence b, KV head kh) before reading
// them: rows b n_q + r (r < n_q) of k_new / v_new, quantised by the append kernel's
// quantisers (NVFP4 groups with the sequence's global scales; K8V4's K rows row-scaled
// FP8) and stored at slots seq_base[b] + L - n_q + r. One thread per (K|V, row, group of
// 16): a row's groups are D/16 consecutive threads. The caller fences before any of its
// loads can touch those slots.
template <int D, int KF>
__device__ inline void append_step_rows(const DecodeParams &p, int b, int kh, int64_t L) {
    constexpr int groups = D / 16;
    const int per_kv = p.n_q * groups;
    for (int t = threadIdx.x; t < 2 * per_kv; t += blockDim.x) {
        const int kv = t >= per_kv;                   // 0 = K, 1 = V
        const int rem = t - kv * per_kv;
        const int r = rem / groups, j = rem - r * groups;
        const int64_t row = (int64_t)b * p.n_q + r;
        const uint16_t *src = (kv ? p.v_new : p.k_new) + (row * p.Hkv + kh) * D + 16 * j;
        const uint4 w0 = *reinterpret_cast<const uint4 *>(src);
        const uint4 w1 = *reinterpret_cast<const uint4 *>(src + 8);
        const uint32_t w[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        const int64_t plane_row = (int64_t)kh * p.cap + p.seq_base[b] + L - p.n_q + r;
        if (KF == 1 && kv == 0) {
            store_fp8_group<D>(w, j, p.kc, p.ks, plane_row);
        } else {
            uint32_t packed[2];
            const uint32_t sc = quantize_group(w, p.gscale[(b * p.Hkv + kh) * 2 + kv], packed);
            *reinterpret_cast<uint2 *>((kv ? p.vc : p.kc) + plane_row * (D / 2) + 8 * j) =
                make_uint2(packed[0], packed[1]);
            (kv ? p.vs : p.ks)[plane_row * groups + j] = (uint8_t)sc;
        }
    }
}

// Query rows of row tile rt -> fp16 MFMA B-fragments in LDS, run by one wave in two
// steps: q_load issues the row loads (before the first KV block's loads, so waiting for
// Q does not wait for KV), q_store converts and stores.
// Fragment (rt, kk, lane (g, n)) = row 16 rt + n, d in [D/4 g + 8 kk, D/4 g + 8 kk + 8).
// Each row is scaled by an exact power of two that brings its maximum magnitude to
// [2^14, 2^15) before the fp16 conversion; sm_c[row] receives the factor that turns an
// MFMA score back into sm_scale * q . k_hat * log2(e) (including the 2^8 of the
// dequantised K and g_K). The factor is kept positive: the sign of sm_scale goes into
// the fragments (an exact negation), and a zero factor (g_K = 0, sm_scale = 0, rows past
// R, whose fragments are zero) becomes kMinScoreScale, which leaves every finite score
// within 2^-72 of 0 and keeps a masked score (-inf) at -inf. Rows past R get zero
// fragments.
template <int D>
__device__ inline void q_load(const DecodeParams &p, const Rows &rw, int b, int kh, int rt, int lane,
                              uint32_t (&w)[D / 8]) {
    constexpr int KK = D / 32;
    constexpr int QD = D / 4;
    const int n = lane & 15, g = lane >> 4;
    const int row = 16 * rt + n;
    if (row < rw.Rc) {
        const int grow = rw.row0 + row;                // row of the KV head's G n_q rows
        const int i = grow / p.G;
        const int h = kh * p.G + (grow - i * p.G);
        const uint16_t *qr = p.q + (((int64_t)b * p.n_q + i) * p.Hq + h) * D + QD * g;
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const uint4 v = *reinterpret_cast<const uint4 *>(qr + 8 * kk);
            w[4 * kk] = v.x; w[4 * kk + 1] = v.y; w[4 * kk + 2] = v.z; w[4 * kk + 3] = v.w;
        }
    } else {
#pragma unroll
        for (int k = 0; k < KK * 4; ++k) w[k] = 0u;
    }
}

template <int D, int KF>
__device__ inline void q_store(const DecodeParams &p, const Rows &rw, int b, int kh, int rt, int lane,
                               const uint32_t (&w)[D / 8], half8_t *qlds, float *sm_c) {
    constexpr int KK = D / 32;
    const int n = lane & 15, g = lane >> 4;
    const int row = 16 * rt + n;
    uint32_t am = 0;
#pragma unroll
    for (int k = 0; k < KK * 4; ++k) am = max(am, max(w[k] & 0x7FFFu, (w[k] >> 16) & 0x7FFFu));
    am = max(am, (uint32_t)__shfl_xor((int)am, 16));
    am = max(am, (uint32_t)__shfl_xor((int)am, 32));
    const int e = (int)((am >> 7) & 0xFF) - 127;
    const int shift = am ? min(max(14 - e, -100), 100) : 0;
    const float qs = p.sm_scale < 0.0f ? -ldexpf(1.0f, shift) : ldexpf(1.0f, shift);
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        u32x4_t hv;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t x = w[4 * kk + k];
            const float lo = __builtin_bit_cast(float, x << 16) * qs;
            const float hi = __builtin_bit_cast(float, x & 0xFFFF0000u) * qs;
            hv[k] = as_u32(half2_t{(_Float16)lo, (_Float16)hi});
        }
        qlds[(rt * KK + kk) * 64 + lane] = __builtin_bit_cast(half8_t, hv);
    }
    if (g == 0) {
        // NVFP4 K: MFMA scores are of e2m1 * S * 2^-8 (times g_K); K8V4's FP8 K: of the E4M3
        // values themselves, the row scales multiplied in per key afterwards
        const float gk = KF ? 1.0f : p.gscale[(b * p.Hkv + kh) * 2 + 0];
        const float c = row < rw.Rc ? fabsf(p.sm_scale) * gk * ldexpf(1.0f, (KF ? 0 : 8) - shift) * kLog2e : 0.0f;
        sm_c[row] = fmaxf(c, kMinScoreScale);
    }
}

}  // namespace dev
}  // namespace nvfp4
