// Split-K decode partial for three or four row tiles (33..64 query rows per KV head):
// the wave-pair kernel (gfx950).
//
// It computes what the single-tile kernel computes (gzenz/ninfer page, "Context and
// model": attention over K/V stored as E2M1 codes + E4M3 group-16 scales; knoopx/ninfer
// page, "Capabilities and limits": MTP verification of 1 + 1..5 draft tokens, which
// with the GQA group gives up to 64 rows per KV head): per unit (sequence, KV head,
// token range) and query row, the unnormalised o, the running max m and the sum l.
//
// Why pairs. With R rows, a wave that owns a whole 32-token block holds R x D fp32
// accumulators; at three or four row tiles that leaves one wave per SIMD and the
// compiler moves accumulators between register files every block. Here the two waves
// of a pair share each block:
//   S^T = K . Q^T   wave w (0/1) takes the 16-token tile w of the block, all rows,
//                   full head_dim (same fragment layout as the single-tile kernel);
//   softmax         each wave writes fp16 probabilities of its 16 tokens to LDS against
//                   the pair's running reference m; the row maxima are reduced and
//                   exchanged only in a block where some score passes m by the lazy
//                   margin (then the pair moves m, rescales and rewrites);
//   O += P . V      each wave reads the whole 32-token P (its own and its partner's,
//                   lane for lane: lane (g, n) of wave w holds exactly the k-slots
//                   4 w .. 4 w + 3 of lane (g, n)'s A operand) and multiplies it into
//                   its half of head_dim: output column n of local tile t is
//                   d = (D/16) n + (D/32) w + t, so lane n's V values again sit in one
//                   scale group (a half group: D/64 code bytes per token).
// Dequantisation work per token is that of the single-tile kernel; the accumulators
// per wave are halved. A workgroup holds kPairs = 4 pairs (every pair a CU keeps resident)
// that merge at the end. The two waves of a pair meet through a handshake in LDS (each
// raises its own count once its LDS writes are complete, then waits for its partner's), not
// through workgroup barriers, so a pair never waits for the other pairs. Each pair starts
// with blocks pair and pair + kPairs and then claims the unit's next unclaimed block from a
// counter in LDS, one block ahead of its loads, so pairs that run faster take more blocks
// (the partition, and with it the fp16 rounding reference of each pair, depends on timing:
// results agree to rounding, not bit for bit). Both waves of a pair read the same claims and
// the same reference-update flags, so they always make the same number of handshakes.
#include "decode_common.h"

namespace nvfp4 {
namespace {

using namespace dev;

// LDS words that the partner wave writes while this wave polls them (volatile, and typed
// as LDS so the accesses stay LDS instructions)
typedef volatile __attribute__((address_space(3))) uint32_t lds_vu32;
typedef volatile __attribute__((address_space(3))) uint16_t lds_vu16;

// Polls of a partner's handshake count before a wave gives up waiting. The partner always
// arrives (both waves make the same handshakes, and every wait follows this wave's own
// count), so the bound only keeps a mistake from hanging the device.
constexpr int kHandshakePolls = 1 << 22;

// The reference m of a row moves only when a score passes m + kPairLazy (base 2), so fp16
// probabilities stay below 2^15 (finite: the fp16 maximum is about 2^16) and a unit's reference
// settles after its first blocks: every later move costs the pair an exchange.
constexpr float kPairLazy = 15.0f;

// KF: the K format (0 NVFP4; 1 the row-scaled FP8 E4M3 K of K8V4), see KGeom.
template <int D, int KF>
struct PairRaw {
    static constexpr int KW = KF ? D / 16 : D / 32;   // K code dwords of one 16-token tile per lane
    static constexpr int KS = KF ? 4 : 1;
    uint32_t k[KW];
    uint32_t ks[KS];                            // NVFP4: D/64 K scale bytes; FP8: fp32 row scales of
                                                // tokens 16 w + 4 g + i
    uint32_t v[8];                              // D/64 V code bytes per k-slot token
    uint32_t vs[8];                             // V scale byte per k-slot token
};

template <int D, int KF>
__device__ inline void pair_load_k(PairRaw<D, KF> &r, rsrc_t kc, rsrc_t ks, const Offs &o) {
#pragma unroll
    for (int c = 0; c < PairRaw<D, KF>::KW / 4; ++c) {
        const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(kc, o.kc + 16 * c, 0, kKCodePolicy<KF>);
        r.k[4 * c] = a[0]; r.k[4 * c + 1] = a[1]; r.k[4 * c + 2] = a[2]; r.k[4 * c + 3] = a[3];
    }
    if constexpr (KF == 1) {
        const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(ks, o.ks, 0, kScalePolicy);
        r.ks[0] = b[0]; r.ks[1] = b[1]; r.ks[2] = b[2]; r.ks[3] = b[3];
    } else if constexpr (D == 256) {
        r.ks[0] = __builtin_amdgcn_raw_buffer_load_b32(ks, o.ks, 0, kScalePolicy);
    } else {
        r.ks[0] = __builtin_amdgcn_raw_buffer_load_b16(ks, o.ks, 0, kScalePolicy);
    }
}

// k-slot j of lane group g is token 16 (j >> 2) + 4 g + (j & 3) of the block; the lane
// offsets already hold the 4 g.
template <int D, int KF>
__device__ inline void pair_load_v(PairRaw<D, KF> &r, rsrc_t vc, rsrc_t vs, const Offs &o) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t dtok = 16 * (j >> 2) + (j & 3);
        if constexpr (D == 256)
            r.v[j] = __builtin_amdgcn_raw_buffer_load_b32(vc, o.vc + dtok * (D / 2), 0, kCodePolicy);
        else
            r.v[j] = __builtin_amdgcn_raw_buffer_load_b16(vc, o.vc + dtok * (D / 2), 0, kCodePolicy);
        r.vs[j] = __builtin_amdgcn_raw_buffer_load_b8(vs, o.vs + dtok * (D / 16), 0, kScalePolicy);
    }
}

// Lane part of the byte offsets of wave w's loads, relative to the block's first slot.
template <int D, int KF>
__device__ inline Offs pair_lane_offsets(int w, int g, int n) {
    constexpr int CB = KGeom<D, KF>::CB;
    Offs o;
    o.kc = (uint32_t)((16 * w + n) * CB + (CB / 4) * g);
    o.ks = KF ? (uint32_t)((16 * w + 4 * g) * 4) : (uint32_t)((16 * w + n) * (D / 16) + (D / 64) * g);
    o.vc = (uint32_t)(4 * g * (D / 2) + (D / 32) * n + (D / 64) * w);
    o.vs = (uint32_t)(4 * g * (D / 16) + (D * n) / 256);
    return o;
}

template <int D, int KF>
__device__ inline half8_t pair_dequant_k(const PairRaw<D, KF> &r, int kk) {
    if constexpr (KF == 1) {
        const uint32_t w0 = r.k[2 * kk], w1 = r.k[2 * kk + 1];
        const u32x4_t a = {fp8x2<0>(w0), fp8x2<1>(w0), fp8x2<0>(w1), fp8x2<1>(w1)};
        return __builtin_bit_cast(half8_t, a);
    } else {
        const uint32_t w = r.k[kk];
        const uint32_t sp = scale_pair((r.ks[0] >> (8 * (kk >> 1))) & 0xFFu);
        const u32x4_t a = {hmul2(fp4x2<0>(w), sp), hmul2(fp4x2<1>(w), sp), hmul2(fp4x2<2>(w), sp),
                           hmul2(fp4x2<3>(w), sp)};
        return __builtin_bit_cast(half8_t, a);
    }
}

// V codes of k-slot pairs (2 kp, 2 kp + 1) interleaved nibble-wise: byte b of E holds
// element 2 b of both tokens, byte b of O element 2 b + 1; SP their fp16 scale pair.
struct PairVPrep {
    uint32_t E[4], O[4], SP[4];
};

template <int D, int KF>
__device__ inline void pair_v_prep(PairVPrep &vp, const PairRaw<D, KF> &r) {
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) {
        const uint32_t wa = r.v[2 * kp], wb = r.v[2 * kp + 1];
        vp.E[kp] = bfi(0x0F0F0F0Fu, wa, wb << 4);
        vp.O[kp] = bfi(0x0F0F0F0Fu, wa >> 4, wb);
        // bit 7 cleared: bytes read past a sequence's end must stay finite (p = 0 there)
        vp.SP[kp] = ((r.vs[2 * kp] & 0x7Fu) << 7) | ((r.vs[2 * kp + 1] & 0x7Fu) << 23);
    }
    // materialise here so the raw V words die before the next block's V loads
#pragma unroll
    for (int kp = 0; kp < 4; ++kp) asm volatile("" : "+v"(vp.E[kp]), "+v"(vp.O[kp]), "+v"(vp.SP[kp]));
}

template <int D, int NT>
struct PairLds {
    static constexpr int KK = D / 32;
    static constexpr int HT = D / 32;                              // PV tiles per wave
    static constexpr int Q_BYTES = NT * KK * 64 * 16;              // Q fragments [NT][KK][lane]
    static constexpr int MERGE_BYTES = 2 * HT * 64 * 16;           // one row tile of both halves
    static constexpr int BIG = Q_BYTES > MERGE_BYTES ? Q_BYTES : MERGE_BYTES;
};

template <int D, int NT, bool DevLen, int KF>
__global__ __attribute__((amdgpu_flat_work_group_size(128 * decode_pairs_per_wg(NT), 128 * decode_pairs_per_wg(NT)),
                          amdgpu_waves_per_eu(decode_waves_per_simd(NT))))
void decode_pair_kernel(DecodeParams p) {
    constexpr int kPairs = decode_pairs_per_wg(NT);               // wave pairs per workgroup
    constexpr int KK = D / 32;
    constexpr int HT = D / 32;          // PV output tiles per wave (half of D/16)
    constexpr int EPL = D / 16;
    using LD = PairLds<D, NT>;
    __shared__ __attribute__((aligned(16))) uint8_t big[LD::BIG];
    __shared__ __attribute__((aligned(16))) u32x4_t pbuf[kPairs][2][NT][64];   // [pair][parity]: fp16 P per lane
    __shared__ float xmax[kPairs][2][NT * 16];                            // [pair][half]
    __shared__ __attribute__((aligned(8))) uint8_t mflag[2][8];           // [parity][wave]
    __shared__ uint32_t ready[2 * kPairs];                                // per wave: handshakes made
    __shared__ uint32_t next_blk;                                         // the unit's next unclaimed block
    __shared__ int claim_buf[kPairs][2];                                  // [pair][parity]: claimed block
    __shared__ float sm_c[kMaxRows];
    __shared__ float sm_m[kPairs][kMaxRows];
    __shared__ float sm_l[kPairs][kMaxRows];

    const int u = blockIdx.x;
    Unit un = unit_of<DevLen>(p, u);
    const Rows rw = rows_of(p);
    trim_causal(un, p, rw);
    const int b = un.b, kh = un.kh, nblk = un.nblk;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int pair = wave >> 1, w = wave & 1;
    const int lane = threadIdx.x & 63, n = lane & 15, g = lane >> 4;
    // R: this launch's rows [row0, row0 + R) of the KV head's Rt = G n_q rows
    const int R = rw.Rc, G = p.G, Rt = p.R, row0 = rw.row0;
    const uint32_t code_bytes = (uint32_t)(p.cap * (D / 2)), scale_bytes = (uint32_t)(p.cap * (D / 16));
    const uint32_t kcode_bytes = (uint32_t)(p.cap * KGeom<D, KF>::CB);
    const uint32_t kscale_bytes = (uint32_t)(p.cap * KGeom<D, KF>::SB);
    const rsrc_t kc = plane_rsrc(p.kc + (int64_t)kh * kcode_bytes, kcode_bytes);
    const rsrc_t ks = plane_rsrc(p.ks + (int64_t)kh * kscale_bytes, kscale_bytes);
    const rsrc_t vc = plane_rsrc(p.vc + (int64_t)kh * code_bytes, code_bytes);
    const rsrc_t vs = plane_rsrc(p.vs + (int64_t)kh * scale_bytes, scale_bytes);
    half8_t *qlds = reinterpret_cast<half8_t *>(big);
    const Offs sentinel{kPastPlane, kPastPlane, kPastPlane, kPastPlane};

    // Q row loads first, then the pair's first block: both latencies overlap, and the Q
    // conversion waits only for Q (vector-memory waits are in order).
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
    int kb = pair;
    const Offs lo = pair_lane_offsets<D, KF>(w, g, n);
    const uint32_t slot_unit = (uint32_t)(p.seq_base[b] + un.t0);
    auto offs_for = [&](int blk) -> Offs {
        return blk < nblk ? add_slot<D, KF>(lo, slot_unit + (uint32_t)(kBlockTokens * blk)) : sentinel;
    };
    PairRaw<D, KF> r;
    {
        const Offs o0 = offs_for(kb);
        pair_load_k<D, KF>(r, kc, ks, o0);
        pair_load_v<D, KF>(r, vc, vs, o0);
    }
    if (wave < NT) q_store<D, KF>(p, rw, b, kh, wave, lane, qw, qlds, sm_c);
    if (threadIdx.x < 16) (&mflag[0][0])[threadIdx.x] = 0;
    if (threadIdx.x < 2 * kPairs) ready[threadIdx.x] = 0;
    if (threadIdx.x == 0) next_blk = 2 * kPairs;
    __syncthreads();
    // Pair handshake: once this wave's LDS accesses are complete it raises its count, then
    // waits for its partner's count to reach the same value.
    uint32_t hs = 0;
    auto pair_sync = [&]() __attribute__((always_inline)) {
        hs += 1;
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (lane == 0) *(lds_vu32 *)&ready[wave] = hs;
        for (int it = 0; it < kHandshakePolls; ++it) {
            const uint32_t o = __builtin_amdgcn_readfirstlane(*(lds_vu32 *)&ready[wave ^ 1]);
            if (o >= hs) break;
            __builtin_amdgcn_s_sleep(1);
        }
        asm volatile("" ::: "memory");
    };
    float cexp[NT];
    int qi[NT];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        const int row = 16 * rt + n;
        cexp[rt] = sm_c[row];
        qi[rt] = row < R ? (row0 + row) / G : p.n_q;  // padded rows see every key (their q is 0)
    }
    // At three row tiles the first tile's Q fragments stay in registers (KK x 4 VGPRs, room
    // left at two waves per SIMD with NVFP4 K): a third less LDS read traffic in the score
    // stage, where the eight waves of the CU otherwise queue on LDS together.
    constexpr int kQReg = (NT == 3 && KF == 0) ? 1 : 0;
    half8_t qreg[kQReg ? KK : 1];
#pragma unroll
    for (int kk = 0; kk < (kQReg ? KK : 0); ++kk) qreg[kk] = qlds[kk * 64 + lane];

    float4_t acc[NT][HT];    // rows 16 rt + 4 g + i, d = EPL n + HT w + t
    float4_t lsum[NT];       // wave 0 of the pair: P . 1 over the same rows
    float m[NT];             // pair-wide reference of row 16 rt + n (base 2)
    float thr[NT];           // m + kPairLazy: a score above it moves the reference
    // -m, or 0 while m = -inf (the exponent offset of P); kept at three row tiles, formed per
    // block at four (where NT more live registers would spill)
    constexpr bool kKeepNmu = NT < 4;
    float nmu[kKeepNmu ? NT : 1];
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        m[rt] = -INFINITY;
        thr[rt] = -INFINITY;
        if constexpr (kKeepNmu) nmu[rt] = 0.0f;
        lsum[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < HT; ++t) acc[rt][t] = float4_t{0.f, 0.f, 0.f, 0.f};
    }
    const half8_t ones = __builtin_bit_cast(half8_t, u32x4_t{0x3C003C00u, 0x3C003C00u, 0x3C003C00u, 0x3C003C00u});

    // The pair's blocks: pair, pair + kPairs, then the blocks it claims. Probabilities are written
    // speculatively: right after its scores, each wave turns block j's scores into fp16
    // P = 2^(x - m) with the reference m it holds, stores them (LDS, parity j & 1) and
    // raises its byte in mflag[j & 1] if any score lies above m + kPairLazy. After the
    // handshake both waves read both bytes, so the decision is the pair's:
    //   none raised (the common case once the first block has set m): P(j) in LDS is final
    //     and O += P(j) . V(j) follows at once -- no row maximum is reduced or exchanged;
    //   some raised: the pair reduces its rows' maxima of block j, exchanges them through
    //     LDS (handshake), moves m where it is exceeded by more than kPairLazy, rescales O and
    //     l, rewrites P(j) (handshake) -- exactly the update a per-block exchange would make,
    //     so the result does not depend on which path ran.
    // One loop trip: handshake -> [update] -> O += P(j) . V(j); V(j + 1) interleave, V(j + 2)
    // loads; S^T(j + 1), K(j + 2) loads, P(j + 1) and its flag, the claim of block j + 3.
    // Double buffers (P, flags, claims by parity of j) are safe: a wave rewrites parity j & 1
    // only after the handshake of trip j + 1, which its partner reaches after its last read
    // of that parity in trip j.
    // lim: offset limit of the block relative to L - n_q (32-bit: tokens < 2^31).
    const int lim0 = (int)(un.L - p.n_q - un.t0);
    // Raw MFMA scores of this wave's 16 tokens (masked: -inf). The score factor c is
    // positive (q_store), so the lane's maximum scaled score is c times max4(x).
    float x[NT][4];

    // fp16 probabilities P = 2^(c s - m) of this wave's 16 tokens of block j into LDS
    auto write_p = [&](int j) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            float nm;
            if constexpr (kKeepNmu) nm = nmu[rt];
            else nm = m[rt] == -INFINITY ? 0.0f : -m[rt];
            const half2_t p01 = half2_t{(_Float16)__builtin_amdgcn_exp2f(fmaf(x[rt][0], cexp[rt], nm)),
                                        (_Float16)__builtin_amdgcn_exp2f(fmaf(x[rt][1], cexp[rt], nm))};
            const half2_t p23 = half2_t{(_Float16)__builtin_amdgcn_exp2f(fmaf(x[rt][2], cexp[rt], nm)),
                                        (_Float16)__builtin_amdgcn_exp2f(fmaf(x[rt][3], cexp[rt], nm))};
            uint32_t *dst = reinterpret_cast<uint32_t *>(&pbuf[pair][j & 1][rt][lane]) + 2 * w;
            typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
            *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{as_u32(p01), as_u32(p23)};
        }
    };

    // S^T of the pair's block j (unit block bj) from the K words in r, the K loads of the
    // next block (bnext), the claim of block j + 2 (wave 0 of the pair), the block's masked
    // scores, its speculative probabilities and this wave's flag.
    auto start_block = [&](int j, int bj, int bnext) __attribute__((always_inline)) {
        asm volatile("" ::: "memory");     // Q fragments are re-read from LDS every block
        float4_t s[NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) s[rt] = float4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kk = 0; kk < KK; ++kk) {
            const half8_t a = pair_dequant_k<D, KF>(r, kk);
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
                s[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, rt < kQReg ? qreg[kk] : qlds[(rt * KK + kk) * 64 + lane],
                                                               s[rt], 0, 0, 0);
        }
        if constexpr (KF == 1) {
            // the keys' row scales (score element i is token 16 w + 4 g + i), taken before the
            // next block's K loads reuse these registers
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i) s[rt][i] *= __builtin_bit_cast(float, r.ks[i]);
        }
        pair_load_k<D, KF>(r, kc, ks, offs_for(bnext));
        if (w == 0 && lane == 0) claim_buf[pair][j & 1] = (int)atomicAdd(&next_blk, 1u);
        const int lim = lim0 - kBlockTokens * bj;
#pragma unroll
        for (int rt = 0; rt < NT; ++rt)
#pragma unroll
            for (int i = 0; i < 4; ++i) x[rt][i] = s[rt][i];
        if (lim < kBlockTokens - 1) {
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (16 * w + 4 * g + i > lim + qi[rt]) x[rt][i] = -INFINITY;
        }
        bool above = false;
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) above |= max4(x[rt]) * cexp[rt] > thr[rt];
        write_p(j);
        const uint8_t flag = __builtin_amdgcn_ballot_w64(above) != 0 ? 1 : 0;   // all lanes vote
        if (lane == 0) mflag[j & 1][wave] = flag;
    };

    // The reference update for block j (both waves of the pair, see above).
    auto update = [&](int j) __attribute__((always_inline)) {
        float mloc[NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            mloc[rt] = wave_max_g(max4(x[rt]) * cexp[rt]);
            if (g == 0) xmax[pair][w][16 * rt + n] = mloc[rt];
        }
        pair_sync();
        bool need_any = false;
        float alpha[NT];
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) {
            const float mb = fmaxf(mloc[rt], xmax[pair][1 - w][16 * rt + n]);
            const bool need = mb > m[rt] + kPairLazy;   // both waves of the pair see the same values
            const float mnew = need ? mb : m[rt];
            alpha[rt] = need ? exp2f(m[rt] - mnew) : 1.0f;   // m = -inf -> 0
            m[rt] = mnew;
            thr[rt] = mnew + kPairLazy;
            if constexpr (kKeepNmu) nmu[rt] = mnew == -INFINITY ? 0.0f : -mnew;
            need_any |= need;
        }
        if (__builtin_amdgcn_ballot_w64(need_any) != 0) {
#pragma unroll
            for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float ai = __shfl(alpha[rt], 4 * g + i);   // accumulator row 4 g + i
                    lsum[rt][i] *= ai;
#pragma unroll
                    for (int t = 0; t < HT; ++t) acc[rt][t][i] *= ai;
                }
            }
        }
        write_p(j);
        pair_sync();
    };

    // O += P(j) . V(j) over this wave's half of head_dim, P(j) of both waves from LDS.
    auto read_p = [&](int j, half8_t (&pa)[NT]) __attribute__((always_inline)) {
#pragma unroll
        for (int rt = 0; rt < NT; ++rt) pa[rt] = __builtin_bit_cast(half8_t, pbuf[pair][j & 1][rt][lane]);
    };
    auto pv_block = [&](const half8_t (&pa)[NT], const PairVPrep &vp) __attribute__((always_inline)) {
#pragma unroll
        for (int t = 0; t < HT; ++t) {
            uint32_t bw[4];
#pragma unroll
            for (int kp = 0; kp < 4; ++kp) {
                const uint32_t src = (t & 1) ? vp.O[kp] : vp.E[kp];
                uint32_t c;
                switch (t >> 1) {
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
                acc[rt][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rt], bh, acc[rt][t], 0, 0, 0);
        }
        if (w == 0) {
#pragma unroll
            for (int rt = 0; rt < NT; ++rt)
                lsum[rt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa[rt], ones, lsum[rt], 0, 0, 0);
        }
    };

    PairVPrep vprep;
    int bj = pair, bj1 = pair + kPairs;    // this pair's blocks j and j + 1
    auto trip = [&](int j) __attribute__((always_inline)) {
        pair_sync();                       // P(j), the flags and the claim of both waves
        const int bj2 = __builtin_amdgcn_readfirstlane((int)*(lds_vu32 *)&claim_buf[pair][j & 1]);
        const uint32_t flags = __builtin_amdgcn_readfirstlane((uint32_t)*((lds_vu16 *)&mflag[j & 1][0] + pair));
        half8_t pa[NT];
        read_p(j, pa);                     // final unless the update below rewrites P(j)
        if (flags != 0) {
            update(j);
            read_p(j, pa);
        }
        pv_block(pa, vprep);
        pair_v_prep<D, KF>(vprep, r);
        __builtin_amdgcn_sched_barrier(0);
        pair_load_v<D, KF>(r, vc, vs, offs_for(bj2));
        if (bj1 < nblk) start_block(j + 1, bj1, bj2);
        bj = bj1;
        bj1 = bj2;
    };

    // A pair's blocks increase (its first two are below every claim), so it is done at its
    // first block past the unit's end.
    if (bj < nblk) {
        start_block(0, bj, bj1);
        pair_v_prep<D, KF>(vprep, r);
        pair_load_v<D, KF>(r, vc, vs, offs_for(bj1));
        for (int j = 0; bj < nblk; ++j) trip(j);
    }

    // ---- merge the two pairs and write the unit's partial
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        if (w == 0 && g == 0) sm_m[pair][16 * rt + n] = m[rt];
        if (w == 0 && n == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) sm_l[pair][16 * rt + 4 * g + i] = lsum[rt][i];
        }
    }
    __syncthreads();                          // also ends every read of the Q fragments
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = 16 * rt + 4 * g + i;
            float M = sm_m[0][row];
#pragma unroll
            for (int q = 1; q < kPairs; ++q) M = fmaxf(M, sm_m[q][row]);
            const float mp = sm_m[pair][row];
            const float f = mp == -INFINITY ? 0.0f : exp2f(mp - M);
#pragma unroll
            for (int t = 0; t < HT; ++t) acc[rt][t][i] *= f;
        }
    }
    // pairs 1 .. kPairs - 1 hand their (rescaled) accumulators to pair 0 in turn, which
    // adds them in that fixed order and writes the unit's partial
    float4_t(*mbuf)[HT][64] = reinterpret_cast<float4_t(*)[HT][64]>(big);   // [role][t][lane]
    float *ws_o = p.ws_o + ((int64_t)u * Rt + row0) * D;
#pragma unroll
    for (int rt = 0; rt < NT; ++rt) {
        for (int q = 1; q < kPairs; ++q) {
            if (pair == q) {
#pragma unroll
                for (int t = 0; t < HT; ++t) mbuf[w][t][lane] = acc[rt][t];
            }
            __syncthreads();
            if (pair == 0) {
#pragma unroll
                for (int t = 0; t < HT; ++t) acc[rt][t] += mbuf[w][t][lane];
            }
            __syncthreads();
        }
        if (pair == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = 16 * rt + 4 * g + i;
                if (row < R) {
                    float *dst = ws_o + (int64_t)row * D + EPL * n + HT * w;
#pragma unroll
                    for (int t = 0; t < HT; t += 4)
                        *reinterpret_cast<float4_t *>(dst + t) =
                            float4_t{acc[rt][t][i], acc[rt][t + 1][i], acc[rt][t + 2][i], acc[rt][t + 3][i]};
                }
            }
        }
    }
    if ((int)threadIdx.x < R) {
        const int row = threadIdx.x;
        float M = sm_m[0][row];
#pragma unroll
        for (int q = 1; q < kPairs; ++q) M = fmaxf(M, sm_m[q][row]);
        float Ls = 0.f;
#pragma unroll
        for (int q = 0; q < kPairs; ++q) {
            const float mq = sm_m[q][row];
            if (mq != -INFINITY) Ls += exp2f(mq - M) * sm_l[q][row];
        }
        p.ws_m[(int64_t)u * Rt + row0 + row] = M;
        p.ws_l[(int64_t)u * Rt + row0 + row] = Ls;
    }
}

template <int D, int NT, int KF>
hipError_t launch_pair_t(const DecodeParams &p, hipStream_t s) {
    if (p.len_dev != nullptr)
        hipLaunchKernelGGL((decode_pair_kernel<D, NT, true, KF>), dim3(p.units, p.grid_y), dim3(128 * decode_pairs_per_wg(NT)), 0, s, p);
    else
        hipLaunchKernelGGL((decode_pair_kernel<D, NT, false, KF>), dim3(p.units, p.grid_y), dim3(128 * decode_pairs_per_wg(NT)), 0, s, p);
    return hipGetLastError();
}

template <int KF>
hipError_t launch_pair_kf(const DecodeParams &p, int D, int NT, hipStream_t s) {
    if (D == 256) {
        switch (NT) {
            case 3: return launch_pair_t<256, 3, KF>(p, s);
            case 4: return launch_pair_t<256, 4, KF>(p, s);
        }
    } else if (D == 128) {
        switch (NT) {
            case 3: return launch_pair_t<128, 3, KF>(p, s);
            case 4: return launch_pair_t<128, 4, KF>(p, s);
        }
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_decode_pair(const DecodeParams &p, int D, int NT, hipStream_t s) {
    return p.k_fp8 ? launch_pair_kf<1>(p, D, NT, s) : launch_pair_kf<0>(p, D, NT, s);
}

}  // namespace nvfp4
