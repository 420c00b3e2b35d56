// Split-K grouped-query decode attention over the NVFP4 KV pool (gfx950).
//
// What is computed (gzenz/ninfer page, "Context and model": attention reads K/V
// stored as E2M1 codes + E4M3 group-16 scales; knoopx/ninfer page, "Capabilities
// and limits": batched decode of 1-8 requests and MTP verification of 1 + 1..5
// draft tokens): for every query row, softmax(sm_scale * q . k_hat) . v_hat over
// the visible keys, with k_hat = e2m1 * S * g_K and v_hat = e2m1 * S * g_V.
//
// Work decomposition. A unit is (sequence b, KV head kh, token range); one
// workgroup runs one unit, each wave taking whole 32-token blocks: at one row tile
// four waves (one per SIMD) take alternate blocks; at two row tiles eight waves (two
// per SIMD, 256 VGPRs each) claim the unit's blocks one at a time from a counter in
// LDS, since the hardware serves the older wave of a SIMD first and a fixed split
// left the younger ones finishing alone (the partition, and with it the fp16 rounding
// reference of each wave, then depends on timing: results agree to rounding, not bit
// for bit). Every query row that reads KV head kh -- GQA group G times n_q query
// tokens, padded to NT tiles of 16 -- shares each KV block, so a block is loaded
// and dequantised once for all of them. Three or four row tiles go to the
// wave-pair kernel, whose waves split each block.
//
// Per 32-token block and wave (MFMA v_mfma_f32_16x16x32_f16, lane l = 16 g + n):
//   S^T = K . Q^T   A = K (16 tokens x 32 d), B = Q^T (32 d x 16 rows), two token
//                   tiles. Lane (g, n) loads token n's d-range [D/4 g, D/4 (g+1)):
//                   D/8 contiguous code bytes + D/64 scale bytes. The contraction
//                   index d is permuted identically in Q, so no transpose is needed.
//                   Result lane (g, n): tokens 16 mt + 4 g + i, row 16 rt + n.
//   softmax         fp32, base 2, per row (lane column n); the running reference m
//                   is raised lazily (only when a score exceeds it by more than 8,
//                   base 2), tested lane by lane, so the cross-lane row maximum and
//                   the accumulator rescale are both rare.
//   O += P . V      A = P (16 rows x 32 tokens, straight from the S^T layout),
//                   B = V (32 tokens x 16 d). The d index of output column n of
//                   tile dt is EPL n + dt (EPL = D/16), so lane n's B values for
//                   every tile lie in ONE 16-element scale group of each token:
//                   8 (or 4) contiguous code bytes and one scale byte per token.
//                   Codes of two tokens are interleaved nibble-wise (v_bfi) so one
//                   fp4->fp16 convert yields a (token, token) k-pair.
// Dequantisation: v_cvt_scalef32_pk_f16_fp4 (scale 1) gives exact E2M1 in fp16;
// the E4M3 byte shifted left by 7 is the fp16 of S * 2^-8, and one v_pk_mul_f16
// forms e2m1 * S * 2^-8 exactly (at most 6 significant bits, >= 2^-18). The 2^8
// and g factors are folded into the score scale and the final output scale.
// Q rows are converted to fp16 after an exact power-of-two scaling that brings
// the row maximum to [2^14, 2^15).
//
// Each workgroup merges its four waves' (o, m, l) through LDS and writes one
// partial per unit; the combine kernel merges the units of a (sequence, head)
// by log-sum-exp in a fixed order (deterministic: no atomics).
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>

#include "decode_common.h"

namespace nvfp4 {
namespace {

using namespace dev;

// KF: the K format (0 NVFP4; 1 the row-scaled FP8 E4M3 K of K8V4), see KGeom.
template <int D, int KF>
struct Raw {
    static constexpr int EPL = D / 16;            // PV output tiles; d-values per token per lane
    static constexpr int KW = KF ? D / 16 : D / 32;   // K code dwords per token per lane
    static constexpr int KS = KF ? 4 : 1;         // K scale dwords per tile per lane
    static constexpr int VW = EPL / 8;            // V code dwords per token per lane
    uint32_t k[2][KW];                            // two 16-token tiles
    uint32_t ks[2][KS];                           // NVFP4: the lane's D/64 scale bytes of token n;
                                                  // FP8: fp32 row scales of tokens 16 mt + 4 g + i
    uint32_t v[8][VW];                            // 8 tokens (k-slots) per lane
    uint32_t vs[8];                               // V scale byte per token
};

template <int D, int KF>
__device__ inline Offs lane_offsets(int64_t slot0, int g, int n) {
    constexpr int EPL = D / 16;
    constexpr int CB = KGeom<D, KF>::CB;
    Offs o;
    o.kc = (uint32_t)((slot0 + n) * CB + (CB / 4) * g);
    o.ks = KF ? (uint32_t)((slot0 + 4 * g) * 4) : (uint32_t)((slot0 + n) * (D / 16) + (D / 64) * g);
    o.vc = (uint32_t)((slot0 + 4 * g) * (D / 2) + (EPL / 2) * n);
    o.vs = (uint32_t)((slot0 + 4 * g) * (D / 16) + (EPL * n) / 16);
    return o;
}

// Loads the K block at o: PART 0 everything; PART 1 the codes of tile 0 only; PART 2 the
// codes of tile 1 and the scales of both tiles.
// Stream: the code loads carry the streaming policy (see kCodePolicy); row chunks side by
// side (grid y > 1) read each block several times and keep the default policy instead.
template <int D, int KF, int PART = 0, bool Stream = true>
__device__ inline void load_k(Raw<D, KF> &r, rsrc_t kc, rsrc_t ks, const Offs &o) {
    constexpr int CB = KGeom<D, KF>::CB, SB = KGeom<D, KF>::SB;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
        const uint32_t oc = o.kc + 16 * mt * CB;
        const uint32_t os = o.ks + 16 * mt * SB;
        if (PART == 0 || PART == mt + 1) {
#pragma unroll
            for (int c = 0; c < Raw<D, KF>::KW / 4; ++c) {
                const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(kc, oc + 16 * c, 0, Stream ? kKCodePolicy<KF> : 0);
                r.k[mt][4 * c] = a[0]; r.k[mt][4 * c + 1] = a[1]; r.k[mt][4 * c + 2] = a[2]; r.k[mt][4 * c + 3] = a[3];
            }
        }
        if (PART == 1) continue;
        if constexpr (KF == 1) {
            const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(ks, os, 0, kScalePolicy);
            r.ks[mt][0] = b[0]; r.ks[mt][1] = b[1]; r.ks[mt][2] = b[2]; r.ks[mt][3] = b[3];
        } else if constexpr (D == 256) {
            r.ks[mt][0] = __builtin_amdgcn_raw_buffer_load_b32(ks, os, 0, kScalePolicy);
        } else {
            r.ks[mt][0] = __builtin_amdgcn_raw_buffer_load_b16(ks, os, 0, kScalePolicy);
        }
    }
}

template <int D, int KF, bool Stream = true>
__device__ inline void load_v(Raw<D, KF> &r, rsrc_t vc, rsrc_t vs, const Offs &o) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t dtok = 16 * (j >> 2) + (j & 3);
        if constexpr (D == 256) {
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t a = __builtin_amdgcn_raw_buffer_load_b64(vc, o.vc + dtok * (D / 2), 0, Stream ? kCodePolicy : 0);
            r.v[j][0] = a[0]; r.v[j][1] = a[1];
        } else {
            r.v[j][0] = __builtin_amdgcn_raw_buffer_load_b32(vc, o.vc + dtok * (D / 2), 0, Stream ? kCodePolicy : 0);
        }
        r.vs[j] = __builtin_amdgcn_raw_buffer_load_b8(vs, o.vs + dtok * (D / 16), 0, kScalePolicy);
    }
}

template <int D, int NT>
struct State {
    static constexpr int EPL = D / 16;
    float4_t acc[NT][EPL];   // O rows 16 rt + 4 g + i, d = EPL n + dt
    float4_t lsum[NT];       // row sums of the fp16 P actually multiplied into O (P . 1), same rows
    float m[NT];             // running reference of row 16 rt + n (base 2)
    float nmu[NT];           // -m, or 0 while m = -inf (the exponent offset of P)
    float thr[NT];           // m + kLazyMax: a block maximum above it moves m
};

// K fragment kk of tile mt: the lane's elements [8 kk, 8 kk + 8) of its d-range, in fp16.
// NVFP4: e2m1 * S * 2^-8 (exact); FP8: the E4M3 values (exact), row scale applied later.
template <int D, int KF>
__device__ inline half8_t dequant_k(const Raw<D, KF> &r, int mt, int kk) {
    if constexpr (KF == 1) {
        const uint32_t w0 = r.k[mt][2 * kk], w1 = r.k[mt][2 * kk + 1];
        const u32x4_t a = {fp8x2<0>(w0), fp8x2<1>(w0), fp8x2<0>(w1), fp8x2<1>(w1)};
        return __builtin_bit_cast(half8_t, a);
    } else {
        const uint32_t w = r.k[mt][kk];
        const uint32_t sp = scale_pair((r.ks[mt][0] >> (8 * (kk >> 1))) & 0xFFu);
        const u32x4_t a = {hmul2(fp4x2<0>(w), sp), hmul2(fp4x2<1>(w), sp), hmul2(fp4x2<2>(w), sp),
                           hmul2(fp4x2<3>(w), sp)};
        return __builtin_bit_cast(half8_t, a);
    }
}

// S^T tiles for the block: s[mt][rt] lane (g, n) = scores of tokens 16 mt + 4 g + i, row 16 rt + n.
template <int D, int NT, int KF>
__device__ inline void qk_block(float4_t (&s)[2][NT], const Raw<D, KF> &r, const half8_t *qlds, int lane) {
    constexpr int KK = D / 32;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) s[mt][rt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kk = 0; kk < KK; ++kk) {
        const half8_t a0 = dequant_k<D, KF>(r, 0, kk);
        const half8_t a1 = dequant_k<D, KF>(r, 1, kk);
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            const half8_t qf = qlds[(rt * KK + kk) * 64 + lane];
            s[0][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, qf, s[0][rt], 0, 0, 0);
            s[1][rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, qf, s[1][rt], 0, 0, 0);
        }
    }
    if constexpr (KF == 1) {
        // the keys' row scales (score element i of tile mt is token 16 mt + 4 g + i); taken
        // before the next block's K loads reuse these registers
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[mt][rt][i] *= __builtin_bit_cast(float, r.ks[mt][i]);
    }
}

// V codes of token pairs (k-slots 2kp, 2kp+1) interleaved nibble-wise, and their scale pairs.
template <int D>
struct VPrep {
    static constexpr int VW = D / 128;
    uint32_t E[4][VW], O[4][VW], SP[4];
};

template <int D, int KF>
__device__ inline void v_prep(VPrep<D> &vp, const Raw<D, KF> &r) {
    constexpr int VW = D / 128;
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
#pragma unroll
        for (int h = 0; h < VW; ++h) {
            const uint32_t wa = r.v[2 * kp][h], wb = r.v[2 * kp + 1][h];
            vp.E[kp][h] = bfi(0x0F0F0F0Fu, wa, wb << 4);   // byte b: (A elem 2b, B elem 2b)
            vp.O[kp][h] = bfi(0x0F0F0F0Fu, wa >> 4, wb);   // byte b: (A elem 2b+1, B elem 2b+1)
        }
        // bit 7 cleared: stored scales never have it; bytes read past a sequence's end
        // (masked, p = 0) must stay finite so 0 * v stays 0.
        vp.SP[kp] = ((r.vs[2 * kp] & 0x7Fu) << 7) | ((r.vs[2 * kp + 1] & 0x7Fu) << 23);
    }
    // Materialise the interleaved words here: otherwise they are computed next to their
    // use in the PV step, the raw V words stay live across the next block's V loads, and
    // those loads need fresh registers plus copies (and a wait) at the loop end.
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
#pragma unroll
        for (int h = 0; h < VW; ++h) asm volatile("" : "+v"(vp.E[kp][h]), "+v"(vp.O[kp][h]));
        asm volatile("" : "+v"(vp.SP[kp]));
    }
}

// Scores -> probabilities for one block. lim = L - n_q - tb: key at offset o of the
// block is visible to query token i iff o <= lim + i (bottom-right causal; offsets
// past the sequence end are never visible). Blocks with lim >= 31 need no mask; the
// mask is applied in place to the raw MFMA scores (masked: -inf).
//
// The scaled score of key j in row r is x = c_r s_j with c_r > 0 (q_store keeps it
// positive), so max_j x = c_r max_j s_j (rounding is monotone). The reference m of a row
// moves only when its block maximum passes m + kLazyMax; that is tested lane by lane
// first (each lane holds 8 of the row's 32 keys), and only when some lane passes does
// the wave reduce the row maxima across lanes and move m -- the same decisions, and the
// same m, as a reduction in every block. P = 2^(c s - m) takes one fma per score.
template <int D, int NT>
__device__ inline void softmax_block(State<D, NT> &st, const float4_t (&s)[2][NT], half8_t (&pa)[NT],
                                     const float (&cexp)[NT], const int (&qi)[NT], int lim, int g) {
    constexpr int EPL = D / 16;
    float x[NT][8];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
#pragma unroll
        for (int j = 0; j < 8; ++j) x[rt][j] = s[j >> 2][rt][j & 3];
    if (lim < kBlockTokens - 1) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int o = 16 * (j >> 2) + 4 * g + (j & 3);
                if (o > lim + qi[rt]) x[rt][j] = -INFINITY;
            }
    }
    float lmax[NT];
    bool above = false;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        lmax[rt] = max8(x[rt]) * cexp[rt];
        above |= lmax[rt] > st.thr[rt];
    }
    if (__builtin_amdgcn_ballot_w64(above) != 0) {   // rare after the first block
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            const float mrow = wave_max_g(lmax[rt]);
            const bool need = mrow > st.thr[rt];
            const float mnew = need ? mrow : st.m[rt];
            const float alpha = need ? exp2f(st.m[rt] - mnew) : 1.0f;   // m = -inf -> 0
            st.m[rt] = mnew;
            st.nmu[rt] = mnew == -INFINITY ? 0.0f : -mnew;
            st.thr[rt] = mnew + kLazyMax;
            // accumulator rows 4 g + i live in lane column n' = 4 g + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * g + i);
                st.lsum[rt][i] *= ai;
#pragma unroll
                for (int dt = 0; dt < EPL; ++dt) st.acc[rt][dt][i] *= ai;
            }
        }
    }
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf(x[rt][j], cexp[rt], st.nmu[rt]));   // v_exp_f32
        pa[rt] = half8_t{(_Float16)p[0], (_Float16)p[1], (_Float16)p[2], (_Float16)p[3],
                         (_Float16)p[4], (_Float16)p[5], (_Float16)p[6], (_Float16)p[7]};
    }
}

template <int D, int NT>
__device__ inline void pv_block(State<D, NT> &st, const VPrep<D> &vp, const half8_t (&pa)[NT]) {
    constexpr int EPL = D / 16;
#pragma unroll
    for (int dt = 0; dt < EPL; ++dt) {
        const int h = dt >> 3, byte = (dt & 7) >> 1;
        uint32_t bw[4];
#pragma unroll
        for (int kp = 0; kp < 4; ++kp) {
            const uint32_t src = (dt & 1) ? vp.O[kp][h] : vp.E[kp][h];
            uint32_t c;
            switch (byte) {
                case 0: c = fp4x2<0>(src); break;
                case 1: c = fp4x2<1>(src); break;
                case 2: c = fp4x2<2>(src); break;
                default: c = fp4x2<3>(src); break;
            }
            bw[kp] = hmul2(c, vp.SP[kp]);
        }
        const half8_t bh = __builtin_bit_cast(half8_t, u32x4_t{bw[0], bw[1], bw[2], bw[3]});
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
            st.acc[rt][dt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rt], bh, st.acc[rt][dt], 0, 0, 0);
    }
    // l from the same fp16 P through the matrix core: P . 1 (fp16 1.0 = 0x3C00)
    const half8_t ones = __builtin_bit_cast(half8_t, u32x4_t{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});
#pragma unroll
    for (int rt = 0; rt < NT; ++rt)
        st.lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rt], ones, st.lsum[rt], 0, 0, 0);
}

template <int D, int NT, int W>
struct Lds {
    static constexpr int KK = D / 32;
    static constexpr int Q_BYTES = NT * KK * 64 * 16;          // Q fragments [NT][KK][lane]
    static constexpr int MERGE_BYTES = W * (D / 16) * 64 * 16; // one row tile of every wave
    static constexpr int BYTES = Q_BYTES > MERGE_BYTES ? Q_BYTES : MERGE_BYTES;
};

template <int D, int NT, bool DevLen, int KF, bool Stream>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * decode_partial_waves(NT), 64 * decode_partial_waves(NT)),
                          amdgpu_waves_per_eu(decode_waves_per_simd(NT))))
void decode_partial_kernel(DecodeParams p) {
    constexpr int EPL = D / 16;
    constexpr int W = decode_partial_waves(NT);
    constexpr bool kClaim = NT == 2;       // waves claim blocks (else a fixed stride of W)
    using LD = Lds<D, NT, W>;
    __shared__ __attribute__((aligned(16))) uint8_t lds[LD::BYTES];
    __shared__ float sm_c[kMaxRows];
    __shared__ float sm_m[W][kMaxRows];
    __shared__ float sm_l[W][kMaxRows];
    __shared__ uint32_t next_blk;          // the unit's next unclaimed block (kClaim)

    const int u = blockIdx.x;
    Unit un = unit_of<DevLen>(p, u);
    const Rows rw = rows_of(p);
    trim_causal(un, p, rw);
    const int b = un.b, kh = un.kh, nblk = un.nblk;
    const int64_t L = un.L, t0 = un.t0;

    // wave index is uniform across the wave; readfirstlane lets the compiler keep the
    // block loop on the scalar unit
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    // R: this launch's rows [row0, row0 + R) of the KV head's Rt = G n_q rows
    const int R = rw.Rc, G = p.G, Rt = p.R, row0 = rw.row0;
    const int64_t base = p.seq_base[b];
    constexpr int KCB = KGeom<D, KF>::CB, KSB = KGeom<D, KF>::SB;
    const uint32_t code_bytes = (uint32_t)(p.cap * (D / 2)), scale_bytes = (uint32_t)(p.cap * (D / 16));
    const uint32_t kcode_bytes = (uint32_t)(p.cap * KCB), kscale_bytes = (uint32_t)(p.cap * KSB);
    const rsrc_t kc = plane_rsrc(p.kc + (int64_t)kh * kcode_bytes, kcode_bytes);
    const rsrc_t ks = plane_rsrc(p.ks + (int64_t)kh * kscale_bytes, kscale_bytes);
    const rsrc_t vc = plane_rsrc(p.vc + (int64_t)kh * code_bytes, code_bytes);
    const rsrc_t vs = plane_rsrc(p.vs + (int64_t)kh * scale_bytes, scale_bytes);
    half8_t *qlds = reinterpret_cast<half8_t *>(lds);

    // Q row loads first, then the first block's KV loads: both latencies overlap, and the
    // Q conversion waits only for Q (vector-memory waits are in order).
    uint32_t qw[D / 8];
    if (wave < NT) q_load<D>(p, rw, b, kh, wave, lane, qw);
    // A decode step that appends its own rows: the workgroup of the sequence's last unit
    // (the only one that reads those slots) stores them before issuing any KV load. The
    // workgroup barrier orders the stores before every wave's later loads (workgroup-scope
    // visibility of global memory: all waves share this CU's vector cache).
    if (p.k_new != nullptr && un.last) {
        append_step_rows<D, KF>(p, b, kh, un.L);
        __syncthreads();
    }
    __builtin_amdgcn_sched_barrier(0);
    Raw<D, KF> r;
    int kb = wave;
    const Offs lo = lane_offsets<D, KF>(0, g, n);
    const uint32_t slot_unit = (uint32_t)(base + t0);
    auto offs_of = [&](int blk) -> Offs {
        return blk < nblk ? add_slot<D, KF>(lo, slot_unit + (uint32_t)(kBlockTokens * blk))
                          : Offs{kPastPlane, kPastPlane, kPastPlane, kPastPlane};
    };
    {
        const Offs o0 = offs_of(kb);
        load_k<D, KF, 0, Stream>(r, kc, ks, o0);
        load_v<D, KF, Stream>(r, vc, vs, o0);
    }
    if (kClaim && threadIdx.x == 0) next_blk = W;

    // ---- Q rows -> fp16 fragments in LDS (wave rt converts row tile rt)
    if (wave < NT) q_store<D, KF>(p, rw, b, kh, wave, lane, qw, qlds, sm_c);
    __syncthreads();
    float cexp[NT];
    int qi[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        const int row = 16 * rt + n;
        cexp[rt] = sm_c[row];
        qi[rt] = row < R ? (row0 + row) / G : p.n_q;  // padded rows see every key (their q is 0)
    }

    State<D, NT> st;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        st.m[rt] = -INFINITY;
        st.nmu[rt] = 0.0f;
        st.thr[rt] = -INFINITY;
        st.lsum[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int dt = 0; dt < EPL; ++dt) st.acc[rt][dt] = float4_t{0.f, 0.f, 0.f, 0.f};
    }

    // ---- stream the unit's blocks: wave w takes blocks w, w+4, ...; the next block's K
    // loads are issued once this block's K is in the S^T tiles, its V loads once this
    // block's V codes are interleaved, so they overlap the softmax and PV work.
    // offset limit of the first block of this wave relative to L - n_q (32-bit: tokens < 2^31)
    // Blocks: wave w starts with block w; then, at two row tiles, each wave claims the next
    // unclaimed block (one LDS atomic per block, issued a block ahead of its loads), at one
    // row tile it steps by W (a fixed partition: the result is deterministic).
    while (kb < nblk) {
        asm volatile("" ::: "memory");
        int kn;
        if constexpr (kClaim) {
            uint32_t nx = 0;
            if (lane == 0) nx = atomicAdd(&next_blk, 1u);
            kn = __builtin_amdgcn_readfirstlane((int)nx);
        } else {
            kn = kb + W;
        }
        const Offs on = offs_of(kn);
        const int lim = (int)(L - p.n_q - t0) - kBlockTokens * kb;
        float4_t s[2][NT];
        qk_block<D, NT, KF>(s, r, qlds, lane);
        // FP8 K at two row tiles: the second tile's codes and both tiles' row scales are
        // loaded at the end of the trip, so their 24 registers are free while the scores,
        // probabilities and interleaved V are live (else 256 VGPRs do not hold the loop)
        constexpr bool kSplitK = KF == 1 && NT == 2 && D == 256;
        if constexpr (kSplitK)
            load_k<D, KF, 1, Stream>(r, kc, ks, on);
        else
            load_k<D, KF, 0, Stream>(r, kc, ks, on);
        VPrep<D> vp;
        v_prep<D, KF>(vp, r);
        // keep the V loads below the code interleave, so they land in the registers it
        // has just read instead of fresh ones that must be copied back at the loop end
        __builtin_amdgcn_sched_barrier(0);
        load_v<D, KF, Stream>(r, vc, vs, on);
        half8_t pa[NT];
        softmax_block<D, NT>(st, s, pa, cexp, qi, lim, g);
        pv_block<D, NT>(st, vp, pa);
        if constexpr (kSplitK) load_k<D, KF, 2, Stream>(r, kc, ks, on);
        kb = kn;
    }

    // ---- merge the waves' (o, m, l) and write the unit's partial
    // Lane indices are recomputed here rather than held in registers across the block loop.
    const int mlane = __lane_id(), mg = mlane >> 4, mn = mlane & 15;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        if (mg == 0) sm_m[wave][16 * rt + mn] = st.m[rt];        // m: row 16 rt + n
        if (mn == 0) {                                            // l: rows 16 rt + 4 g + i
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_l[wave][16 * rt + 4 * mg + i] = st.lsum[rt][i];
        }
    }
    __syncthreads();                                  // also ends every read of the Q fragments
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * mg + i;
            float M = -INFINITY;
#pragma unroll
            for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][row]);
            const float mw = sm_m[wave][row];
            const float f = mw == -INFINITY ? 0.0f : exp2f(mw - M);
#pragma unroll
            for (int dt = 0; dt < EPL; ++dt) st.acc[rt][dt][i] *= f;
        }
    }
    // Sum of the W waves' accumulators, one row tile at a time. Each wave stores its tile
    // as EPL float4 rows of 64 lanes (1 KB, lane-contiguous: conflict-free stores), lane L of
    // row dt at slot L ^ dt. A thread then sums the W copies of one (dt, L) float4 -- lanes
    // dt = 0..15 of a 16-lane group read slots L ^ dt, all in different banks -- and
    // stores its 4 rows; for each row a wave's stores cover 64 consecutive floats.
    u32x4_t *mrg = reinterpret_cast<u32x4_t *>(lds);
    float *ws_o = p.ws_o + ((int64_t)u * Rt + row0) * D;
    constexpr int UNITS = EPL * 64;                   // (dt, lane) float4s per wave and tile
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
        for (int dt = 0; dt < EPL; ++dt)
            mrg[(wave * EPL + dt) * 64 + (mlane ^ dt)] = __builtin_bit_cast(u32x4_t, st.acc[rt][dt]);
        __syncthreads();
        for (int e = wave * 64 + mlane; e < UNITS; e += 64 * W) {
            const int dt = e % EPL, L = e / EPL;          // L = 16 g' + n'
            float4_t s = __builtin_bit_cast(float4_t, mrg[dt * 64 + (L ^ dt)]);
#pragma unroll
            for (int w = 1; w < W; ++w) s += __builtin_bit_cast(float4_t, mrg[(w * EPL + dt) * 64 + (L ^ dt)]);
            const int gg = L >> 4, nn = L & 15;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rt + 4 * gg + i;
                if (row < R) ws_o[(int64_t)row * D + EPL * nn + dt] = s[i];
            }
        }
        __syncthreads();
    }
    if (wave * 64 + mlane < R) {
        const int row = wave * 64 + mlane;
        float M = -INFINITY;
        for (int w = 0; w < W; ++w) M = fmaxf(M, sm_m[w][row]);
        float Ls = 0.f;
        for (int w = 0; w < W; ++w) {
            const float mw = sm_m[w][row];
            if (mw != -INFINITY) Ls += exp2f(mw - M) * sm_l[w][row];
        }
        p.ws_m[(int64_t)u * Rt + row0 + row] = M;
        p.ws_l[(int64_t)u * Rt + row0 + row] = Ls;
    }
}

// One 256-thread workgroup per (sequence, KV head, row). Wave w merges units
// w, w + 4, ... of that (sequence, head) with its own running maximum (m, l and o of
// a unit are loaded together, so the merge costs one memory latency, not two); lane c
// owns the D/64 contiguous outputs [c D/64, (c + 1) D/64). The four wave results are
// merged through LDS. Every sum runs in a fixed order, so the result does not depend
// on timing.
// Built for up to 128 VGPRs (four waves per SIMD; the grid is one workgroup per output
// row): at the default target of eight waves the compiler held back three of a batch's
// eight partial loads until the first five had arrived, a second memory round trip. Same
// box: decode_27b step 24.0 -> 23.3 us; at one wave per SIMD the three-session step got
// slower instead (261.5 -> 263.5 us; four waves: 261.1).
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256), amdgpu_waves_per_eu(4, 4)))
void decode_combine_kernel(DecodeParams p) {
    constexpr int PER = D / 64;                       // outputs per lane
    typedef float vecf __attribute__((ext_vector_type(PER)));
    // grid (R, Hkv, B): the indices need no kernel argument, so the per-sequence arguments
    // below are loaded in the kernel's first round of scalar loads
    const int R = p.R;
    const int r = blockIdx.x, kh = blockIdx.y, b = blockIdx.z;
    const int ns = p.n_split[b];
    const int64_t u0 = (int64_t)p.unit_base[b] + (int64_t)kh * ns;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
    const float *gvp = p.gscale + (b * p.Hkv + kh) * 2 + 1;
    const int i = r / p.G, h = kh * p.G + (r - i * p.G);
    const int64_t idx = (((int64_t)b * p.n_q + i) * p.Hq + h) * D + PER * lane;
    uint8_t *const outp = static_cast<uint8_t *>(p.out);
    const int out_bf16 = p.out_bf16;
    const float *mrow = p.ws_m + u0 * R + r;          // m of unit s at mrow[s * R]
    const float *lrow = p.ws_l + u0 * R + r;
    const float *orow = p.ws_o + (u0 * R + r) * D + PER * lane;
    // batches of 8 units: every load of a batch is issued before any of it is used
    constexpr int BATCH = 8;
    // m and l are the same for every lane; an index the compiler cannot prove uniform
    // keeps their loads on the vector path, where a batch's loads go out together (as
    // scalar loads they were issued one after another)
    int vz;
    asm volatile("v_mov_b32 %0, 0" : "=v"(vz));
    float M = -INFINITY, den = 0.f, gv = 0.f;
    vecf acc = {};
    if (ns <= kWaves) {
        // at most one unit per wave (long query chunks split into few units): that unit's
        // loads alone, not a batch of copies of it
        gv = gvp[vz];
        if (wave < ns) {
            M = mrow[(int64_t)wave * R + vz];
            den = lrow[(int64_t)wave * R + vz];
            acc = *reinterpret_cast<const vecf *>(orow + (int64_t)wave * R * D);
        }
        asm volatile("" ::"s"(outp), "s"(out_bf16));
    }
    for (int s0 = wave; ns > kWaves && s0 < ns; s0 += kWaves * BATCH) {
        // g_V and the output's arguments in the batch's round trip rather than after the
        // cross-wave merge (wave 0, which writes the output, always runs this loop)
        gv = gvp[vz];
        float ms[BATCH], ls[BATCH];
        vecf o[BATCH];
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const int s = s0 + k * kWaves;
            const int64_t sc = s < ns ? s : ns - 1;      // past the end: a real unit, weight 0
            ms[k] = mrow[sc * R + vz];
            ls[k] = lrow[sc * R + vz];
            o[k] = *reinterpret_cast<const vecf *>(orow + sc * R * D);
            if (s >= ns) ms[k] = -INFINITY;
        }
        asm volatile("" ::"s"(outp), "s"(out_bf16));
        float mb = ms[0];
#pragma unroll
        for (int k = 1; k < BATCH; ++k) mb = fmaxf(mb, ms[k]);
        const float Mn = fmaxf(M, mb);
        const float f = M == -INFINITY ? 0.0f : exp2f(M - Mn);
        acc *= f;
        den *= f;
        M = Mn;
#pragma unroll
        for (int k = 0; k < BATCH; ++k) {
            const float w = ms[k] == -INFINITY ? 0.0f : exp2f(ms[k] - M);
            acc += w * o[k];
            den += w * ls[k];
        }
    }
    __shared__ vecf part[kWaves][64];
    __shared__ float mpart[kWaves], dpart[kWaves];
    part[wave][lane] = acc;
    if (lane == 0) {
        mpart[wave] = M;
        dpart[wave] = den;
    }
    __syncthreads();
    if (wave == 0) {
        float Mx = mpart[0];
#pragma unroll
        for (int w = 1; w < kWaves; ++w) Mx = fmaxf(Mx, mpart[w]);
        vecf o = {};
        float dd = 0.f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float f = mpart[w] == -INFINITY ? 0.0f : exp2f(mpart[w] - Mx);
            o += f * part[w][lane];
            dd += f * dpart[w];
        }
        // v_hat = (e2m1 * S * 2^-8) * 2^8 * g_V
        o *= 256.0f * gv / dd;
        if (out_bf16) {
            // IEEE conversion: round to nearest even (v_cvt_pk_bf16_f32)
            typedef __bf16 vecb __attribute__((ext_vector_type(PER)));
            vecb ob;
#pragma unroll
            for (int k = 0; k < PER; ++k) ob[k] = (__bf16)o[k];
            *reinterpret_cast<vecb *>(reinterpret_cast<__bf16 *>(outp) + idx) = ob;
        } else {
            *reinterpret_cast<vecf *>(reinterpret_cast<float *>(outp) + idx) = o;
        }
    }
}

template <int D, int NT, int KF, bool Stream>
hipError_t launch_partial_s(const DecodeParams &p, hipStream_t s) {
    if (p.len_dev != nullptr)
        hipLaunchKernelGGL((decode_partial_kernel<D, NT, true, KF, Stream>), dim3(p.units, p.grid_y),
                           dim3(64 * decode_partial_waves(NT)), 0, s, p);
    else
        hipLaunchKernelGGL((decode_partial_kernel<D, NT, false, KF, Stream>), dim3(p.units, p.grid_y),
                           dim3(64 * decode_partial_waves(NT)), 0, s, p);
    return hipGetLastError();
}

// Row chunks side by side (grid y > 1, two row tiles only) read every block once per chunk,
// mostly from cache: default-policy code loads there (same box, A/B in one process: 96 rows
// over 131k tokens 86.7 -> 81.9 us per step, a 1,024-token prefill chunk 926.8 -> 900.8 us).
template <int D, int NT, int KF>
hipError_t launch_partial_t(const DecodeParams &p, hipStream_t s) {
    if constexpr (NT == 2) {
        if (p.grid_y > 1) return launch_partial_s<D, NT, KF, false>(p, s);
    }
    return launch_partial_s<D, NT, KF, true>(p, s);
}

template <int KF>
hipError_t launch_partial_kf(const DecodeParams &p, int D, int NT, hipStream_t s) {
    if (D == 256) return NT == 1 ? launch_partial_t<256, 1, KF>(p, s) : launch_partial_t<256, 2, KF>(p, s);
    if (D == 128) return NT == 1 ? launch_partial_t<128, 1, KF>(p, s) : launch_partial_t<128, 2, KF>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_partial(const DecodeParams &p, int D, int NT, hipStream_t s) {
    if (NT > 2) return launch_decode_pair(p, D, NT, s);
    return p.k_fp8 ? launch_partial_kf<1>(p, D, NT, s) : launch_partial_kf<0>(p, D, NT, s);
}

hipError_t launch_decode_combine(const DecodeParams &p, int D, hipStream_t s) {
    const dim3 blocks((unsigned)p.R, (unsigned)p.Hkv, (unsigned)p.B);
    if (D == 256)
        hipLaunchKernelGGL(decode_combine_kernel<256>, dim3(blocks), dim3(256), 0, s, p);
    else if (D == 128)
        hipLaunchKernelGGL(decode_combine_kernel<128>, dim3(blocks), dim3(256), 0, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace nvfp4
