"""Pins of the oracle's K8V4 path (knoopx/ninfer page, "Capabilities and limits": K8V4 KV
storage, 8-bit K with 4-bit V). Reading: K is row-scaled FP8 E4M3, the engine's 8-bit
format (knoopx/ninfer page, "Performance": "FP8 E4M3 row-256"; gzenz/ninfer page,
"Capabilities and limits": row-scaled FP8 E4M3 KV storage): per (token, KV head) row,
s = fp32(amax_row / 448), code = sign << 7 | E4M3 nearest the exact |x| / s (ties to the
even code, saturating at 448); V is NVFP4.

Pinned by: hand-worked rows (tests/golden), exact-rational brute force of the row scale and
of every code (E4M3 values from torch's float8_e4m3fn decoding, not the oracle's table),
the quantiser's error bound, the packed-size arithmetic, and float64 SDPA over the
dequantised tensors.
"""
import json
import math
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import workloads
from test_oracle_formats import E4M3_POS, brute_nearest_even

HERE = os.path.dirname(os.path.abspath(__file__))


def _bf16(vals):
    out = []
    for v in vals:
        if v == "-0":
            out.append(0x8000)
        else:
            out.append(int(workloads.as_u16(torch.tensor([float(v)], dtype=torch.float32).to(torch.bfloat16))[0]))
    return np.array(out, np.uint16)


def _nearest_fp32_ok(f: float, exact: Fraction) -> bool:
    lo = float(np.nextafter(np.float32(f), np.float32(-np.inf)))
    hi = float(np.nextafter(np.float32(f), np.float32(np.inf)))
    d = abs(Fraction(f) - exact)
    return d <= abs(Fraction(lo) - exact) and d <= abs(Fraction(hi) - exact)


def test_hand_worked_rows():
    gold = json.load(open(os.path.join(HERE, "golden", "k8v4_fp8_row_hand_worked.json")))
    for row in gold["rows"]:
        D = row["head_dim"]
        x = np.zeros(D, np.uint16)
        for idx, val in row["x"]:
            x[idx] = _bf16([val])[0]
        codes, scale = oracle.quantize_rows_fp8(x[None])
        exp = np.zeros(D, np.uint8)
        for idx, c in row["codes"]:
            exp[idx] = c
        np.testing.assert_array_equal(codes[0], exp, err_msg=row["why"])
        s_exact = Fraction(row["scale"])
        assert _nearest_fp32_ok(float(scale[0]), s_exact), (row["scale"], float(scale[0]))
        if s_exact.denominator & (s_exact.denominator - 1) == 0:     # power-of-two denominator: exact
            assert Fraction(float(scale[0])) == s_exact


def _brute_row(x_u16):
    """Expected (codes, scale) of one row by exact rationals, independent of the oracle."""
    xs = workloads.from_u16(x_u16).float().numpy().astype(np.float64)
    amax = max(abs(v) for v in xs)
    s_exact = Fraction(amax) / 448
    s = float(np.float32(float(s_exact)))          # nearest-even fp32 of the rational (checked below)
    assert _nearest_fp32_ok(s, s_exact)
    codes = []
    for u, v in zip(x_u16, xs):
        sign = (int(u) >> 15) & 1
        mag = 0 if s == 0.0 else brute_nearest_even(abs(v), s, E4M3_POS)
        codes.append((sign << 7) | mag)
    return np.array(codes, np.uint8), s


def test_rows_match_exact_rational_bruteforce():
    rng = random.Random(77)
    rows = []
    for D in (128, 256):
        for _ in range(6):                                       # random magnitudes over a wide range
            e = rng.uniform(-12, 12)
            rows.append((D, [rng.gauss(0, 1) * 10 ** e * (10 ** rng.uniform(-3, 0)) for _ in range(D)]))
        for k in (-5, 0, 3):                                     # s = 2^k: every E4M3 midpoint exactly
            mids = [(E4M3_POS[i] + E4M3_POS[i + 1]) / 2 * 2.0 ** k for i in range(126)]
            v = [448 * 2.0 ** k] + mids[:D - 1]
            v += [0.0] * (D - len(v))
            rows.append((D, [(-1) ** i * t for i, t in enumerate(v)]))
    for D, vals in rows:
        x = _bf16(vals)
        codes, scale = oracle.quantize_rows_fp8(x[None])
        exp_codes, exp_s = _brute_row(x)
        assert float(scale[0]) == exp_s
        np.testing.assert_array_equal(codes[0], exp_codes)


def test_error_bound_and_saturation_free_max():
    """|x - x_hat| <= half the E4M3 gap at |x| / s, times s; the row maximum lands within
    E4M3 rounding of 448 s (never above, since amax / s <= 448 (1 + 2^-24))."""
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal(64 * 256) * 3.0).reshape(64, 256)
    codes, scales = oracle.quantize_rows_fp8(x)
    xh = oracle.dequantize_rows_fp8(codes, scales)
    xf = workloads.from_u16(x).double().numpy()
    pos = np.array(E4M3_POS)
    for r in range(64):
        s = float(scales[r])
        v = np.abs(xf[r]) / s
        idx = np.clip(np.searchsorted(pos, v), 1, 126)
        gap = pos[idx] - pos[idx - 1]
        assert np.all(np.abs(xf[r] - xh[r]) <= 0.5 * gap * s * (1 + 1e-12))
        j = int(np.argmax(np.abs(xf[r])))
        assert codes[r, j] & 0x7F == 0x7E


def test_packed_size_arithmetic_k8v4():
    """K8V4 bytes per (token, KV head): K = D codes + one fp32 scale, V = D/2 + D/16 (NVFP4):
    404 at D = 256 (1.578 B per element, against 2 x 0.5625 for NVFP4 K and V)."""
    for D, exp in ((256, 404), (128, 204)):
        c = oracle.Cache(2, D, 10, kv_format="k8v4")
        per = (c.k_codes.nbytes + c.k_scales.nbytes + c.v_codes.nbytes + c.v_scales.nbytes) / (2 * 10)
        assert per == exp
        assert workloads.packed_bytes_per_token_head(D, "k8v4") == exp


@pytest.mark.parametrize("shape", [
    dict(seq_lens=(37,), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=1),
    dict(seq_lens=(50, 19), num_kv_heads=2, num_q_heads=6, head_dim=256, n_q=3, outlier_frac=0.02),
])
def test_k8v4_attention_matches_torch_sdpa_float64(shape):
    w = workloads.small(**shape, kv_format="k8v4")
    k = workloads.all_kv_rows(w, "k")
    v = workloads.all_kv_rows(w, "v")
    ku, vu = workloads.as_u16(k), workloads.as_u16(v)
    g = oracle.calibrate(ku, vu, w.seq_lens)
    cache = oracle.Cache(w.num_kv_heads, w.head_dim, w.capacity, kv_format="k8v4")
    oracle.append(cache, ku, vu, g, w.seq_base, [0] * w.batch, list(w.seq_lens))
    q = workloads.queries(w)
    out = oracle.attention(cache, g, workloads.as_u16(q), w.seq_base, w.seq_lens, w.n_q, w.sm_scale)
    G = w.group
    for b, L in enumerate(w.seq_lens):
        base = w.seq_base[b]
        K = torch.stack([torch.from_numpy(oracle.dequantize_rows_fp8(cache.k_codes[h, base:base + L],
                                                                     cache.k_scales[h, base:base + L]))
                         for h in range(w.num_kv_heads)])
        V = torch.stack([torch.from_numpy(oracle.dequantize_rows(cache.v_codes[h, base:base + L],
                                                                 cache.v_scales[h, base:base + L], g[b, h, 1]))
                         for h in range(w.num_kv_heads)])
        Q = q[b].to(torch.float64).transpose(0, 1)
        mask = torch.zeros(w.n_q, L, dtype=torch.bool)
        for i in range(w.n_q):
            mask[i, :L - w.n_q + i + 1] = True
        ref = torch.nn.functional.scaled_dot_product_attention(Q, K.repeat_interleave(G, 0), V.repeat_interleave(G, 0),
                                                               attn_mask=mask, scale=w.sm_scale)
        got = torch.from_numpy(out[b]).transpose(0, 1)
        assert torch.allclose(got, ref, rtol=1e-12, atol=1e-12)
    # the K rows really are row-scaled FP8: dequantised K differs from the NVFP4 K of the same rows
    c4 = oracle.Cache(w.num_kv_heads, w.head_dim, w.capacity)
    oracle.append(c4, ku, vu, g, w.seq_base, [0] * w.batch, list(w.seq_lens))
    np.testing.assert_array_equal(c4.v_codes, cache.v_codes)
    out4 = oracle.attention(c4, g, workloads.as_u16(q), w.seq_base, w.seq_lens, w.n_q, w.sm_scale)
    assert not np.allclose(out4, out, rtol=0, atol=1e-9)


def test_k8v4_append_places_rows():
    """K8V4 append: K rows quantised row-scaled FP8 at their slots (g_K not used), V NVFP4."""
    rng = np.random.default_rng(21)
    H, D, cap = 2, 128, 32
    k = _bf16(rng.standard_normal(3 * H * D)).reshape(3, H, D)
    v = _bf16(rng.standard_normal(3 * H * D)).reshape(3, H, D)
    g = np.array([[[123.0, 0.001], [7.0, 0.002]]], np.float32)
    cache = oracle.Cache(H, D, cap, kv_format="k8v4")
    oracle.append(cache, k, v, g, [10], [5], [3])
    for r in range(3):
        for h in range(H):
            kc, ks = oracle.quantize_rows_fp8(k[r, h][None])
            np.testing.assert_array_equal(cache.k_codes[h, 15 + r], kc[0])
            assert cache.k_scales[h, 15 + r] == ks[0]
            vc, vs = oracle.quantize_rows(v[r, h][None], g[0, h, 1])
            np.testing.assert_array_equal(cache.v_codes[h, 15 + r], vc[0])
    assert not cache.k_codes[:, :15].any() and not cache.k_scales[:, 18:].any()
