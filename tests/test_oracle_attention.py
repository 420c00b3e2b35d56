"""Oracle attention pins: library reduction, brute-force invariants, causal reduction.

Decode over the NVFP4 KV cache is plain softmax attention over the dequantised
rows (gzenz/ninfer page, "Context and model"; GQA and 1 + draft verify rows
from the knoopx/ninfer page, "Capabilities and limits": MTP draft windows of
one to five, one to eight active requests).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

E4M3_ONE = 0x38        # E4M3 byte of 1.0
E2M1_ONE = 0x2         # E2M1 code of 1.0


def build_cache(w: workloads.Workload):
    """Oracle cache + global scales for a workload, from the shared seeded generators."""
    k = workloads.all_kv_rows(w, "k")
    v = workloads.all_kv_rows(w, "v")
    ku, vu = workloads.as_u16(k), workloads.as_u16(v)
    g = oracle.calibrate(ku, vu, w.seq_lens)
    cache = oracle.Cache(w.num_kv_heads, w.head_dim, w.capacity)
    oracle.append(cache, ku, vu, g, w.seq_base, [0] * w.batch, list(w.seq_lens))
    return cache, g


def dequant_head(cache, g, b, h, base, L, which):
    codes = cache.k_codes if which == "k" else cache.v_codes
    scales = cache.k_scales if which == "k" else cache.v_scales
    return oracle.dequantize_rows(codes[h, base:base + L], scales[h, base:base + L],
                                  g[b, h, 0 if which == "k" else 1])


@pytest.mark.parametrize("shape", [
    dict(seq_lens=(37,), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=1),
    dict(seq_lens=(50, 19), num_kv_heads=2, num_q_heads=6, head_dim=256, n_q=3),
    dict(seq_lens=(64, 6, 33), num_kv_heads=2, num_q_heads=4, head_dim=128, n_q=6, v_dist="laplace"),
])
def test_matches_torch_sdpa_float64(shape):
    w = workloads.small(**shape)
    cache, g = build_cache(w)
    q = workloads.queries(w)
    out = oracle.attention(cache, g, workloads.as_u16(q), w.seq_base, w.seq_lens, w.n_q, w.sm_scale)
    G = w.group
    for b, L in enumerate(w.seq_lens):
        base = w.seq_base[b]
        K = torch.stack([torch.from_numpy(dequant_head(cache, g, b, h, base, L, "k")) for h in range(w.num_kv_heads)])
        V = torch.stack([torch.from_numpy(dequant_head(cache, g, b, h, base, L, "v")) for h in range(w.num_kv_heads)])
        Kq = K.repeat_interleave(G, dim=0)                     # q head h reads kv head h // G
        Vq = V.repeat_interleave(G, dim=0)
        Q = q[b].to(torch.float64).transpose(0, 1)             # [Hq, n_q, D]
        mask = torch.zeros(w.n_q, L, dtype=torch.bool)
        for i in range(w.n_q):
            mask[i, :L - w.n_q + i + 1] = True                 # bottom-right causal
        ref = torch.nn.functional.scaled_dot_product_attention(Q, Kq, Vq, attn_mask=mask, scale=w.sm_scale)
        got = torch.from_numpy(out[b]).transpose(0, 1)
        assert torch.allclose(got, ref, rtol=1e-12, atol=1e-12)


def _const_cache(Hkv, D, cap, k_code=E2M1_ONE, v_code=E2M1_ONE):
    c = oracle.Cache(Hkv, D, cap)
    c.k_codes[:] = k_code | (k_code << 4)
    c.v_codes[:] = v_code | (v_code << 4)
    c.k_scales[:] = E4M3_ONE
    c.v_scales[:] = E4M3_ONE
    return c


def _rand_q(B, n_q, Hq, D, seed=0):
    return workloads.as_u16(torch.randn(B, n_q, Hq, D, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16))


def test_weights_sum_to_one():
    c = _const_cache(2, 128, 40)
    g = np.ones((1, 2, 2), np.float32)
    out = oracle.attention(c, g, _rand_q(1, 3, 4, 128), [0], [40], 3, 0.1)
    assert np.allclose(out, 1.0, rtol=0, atol=1e-15)


def test_single_token_returns_its_v_row():
    w = workloads.small(seq_lens=(1, 1), num_kv_heads=2, num_q_heads=6, head_dim=256, n_q=1)
    cache, g = build_cache(w)
    out = oracle.attention(cache, g, _rand_q(2, 1, 6, 256), w.seq_base, w.seq_lens, 1, w.sm_scale)
    for b in range(2):
        for h in range(6):
            vrow = dequant_head(cache, g, b, h // 3, w.seq_base[b], 1, "v")[0]
            assert np.array_equal(out[b, 0, h], vrow)          # GQA: head h reads kv head h // 3


def test_constant_v_gives_constant_output():
    c = _const_cache(1, 128, 70, k_code=0x5, v_code=0xB)       # K = 3, V = -1.5
    rng = np.random.default_rng(0)
    c.k_codes[:] = rng.integers(0, 256, c.k_codes.shape, dtype=np.uint8)
    g = np.array([[[0.37, 2.0]]], np.float32)
    out = oracle.attention(c, g, _rand_q(1, 2, 4, 128), [0], [70], 2, 0.09)
    assert np.allclose(out, -3.0, rtol=0, atol=1e-14)          # -1.5 * S(1) * g_V(2)


def test_zero_query_gives_mean_of_visible_rows():
    w = workloads.small(seq_lens=(45,), num_kv_heads=1, num_q_heads=2, head_dim=128, n_q=4)
    cache, g = build_cache(w)
    q = np.zeros((1, 4, 2, 128), np.uint16)                    # bf16 +0
    out = oracle.attention(cache, g, q, [0], [45], 4, w.sm_scale)
    V = dequant_head(cache, g, 0, 0, 0, 45, "v")
    for i in range(4):
        assert np.allclose(out[0, i, 0], V[:45 - 4 + i + 1].mean(axis=0), rtol=1e-12, atol=1e-13)


def test_dominant_key_returns_its_row():
    D, L = 128, 30
    c = _const_cache(1, D, L)
    rng = np.random.default_rng(5)
    c.v_codes[:] = rng.integers(0, 256, c.v_codes.shape, dtype=np.uint8)
    c.k_codes[:] = 0                                           # every key 0 ...
    c.k_codes[0, 17] = 0x77                                    # ... except key 17 = +6 everywhere
    g = np.array([[[1.0, 1.0]]], np.float32)
    q = np.full((1, 1, 1, D), 0x3F80, np.uint16)               # bf16 1.0
    out = oracle.attention(c, g, q, [0], [L], 1, 1.0)          # score 768 vs 0
    V = oracle.dequantize_rows(c.v_codes[0], c.v_scales[0], np.float32(1.0))
    assert np.allclose(out[0, 0, 0], V[17], rtol=0, atol=1e-300)


def test_causal_reduction_to_single_query():
    """MTP row i equals an n_q = 1 decode over the first L - n_q + i + 1 keys."""
    w = workloads.small(seq_lens=(90,), num_kv_heads=2, num_q_heads=4, head_dim=256, n_q=5)
    cache, g = build_cache(w)
    q = workloads.as_u16(workloads.queries(w))
    full = oracle.attention(cache, g, q, [0], [90], 5, w.sm_scale)
    for i in range(5):
        one = oracle.attention(cache, g, np.ascontiguousarray(q[:, i:i + 1]), [0], [90 - 5 + i + 1], 1, w.sm_scale)
        assert np.allclose(full[0, i], one[0, 0], rtol=1e-13, atol=1e-14)


def test_selected_rows_match_full():
    w = workloads.small(seq_lens=(40, 25), num_kv_heads=2, num_q_heads=6, head_dim=128, n_q=2)
    cache, g = build_cache(w)
    q = workloads.as_u16(workloads.queries(w))
    full = oracle.attention(cache, g, q, w.seq_base, w.seq_lens, 2, w.sm_scale)
    sel = [(1, 1, 5), (0, 0, 0), (1, 0, 2)]
    part = oracle.attention(cache, g, q, w.seq_base, w.seq_lens, 2, w.sm_scale, sel=sel)
    for n, (b, i, h) in enumerate(sel):
        assert np.array_equal(part[n], full[b, i, h])
