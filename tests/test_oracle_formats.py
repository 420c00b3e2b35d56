"""Pins of the oracle's format arithmetic against things other than itself.

Sources: the NVFP4 KV format is "4-bit E2M1 codes + E4M3 group-16 scales"
(gzenz/ninfer page, section "Context and model"); the size claim "45% less KV
VRAM than int8" is the same bullet. E2M1 and E4M3 are taken as the OCP MX v1.0
element formats (E4M3 = E4M3FN).
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

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "nvfp4_hand_worked.json")

# The E2M1 value set fixed by the format: {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6},
# written out per code (magnitude codes 0..7 in increasing order, bit 3 = sign).
E2M1_BY_CODE = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def torch_e4m3_values():
    """Decoded values of all 256 E4M3FN bytes by torch (a library routine)."""
    b = torch.arange(256, dtype=torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).tolist()


# ---- P1: E2M1 decode ----------------------------------------------------------------------
def test_e2m1_decode_all_codes():
    for code in range(16):
        mag = E2M1_BY_CODE[code & 7]
        v = oracle.e2m1_value(code)
        assert abs(v) == mag
        assert math.copysign(1.0, v) == (-1.0 if code & 8 else 1.0)
    assert sorted({abs(oracle.e2m1_value(c)) for c in range(16)}) == E2M1_BY_CODE


# ---- P2: E4M3 decode ----------------------------------------------------------------------
def test_e4m3_decode_matches_torch_float8_e4m3fn():
    ref = torch_e4m3_values()
    for byte in range(256):
        v = oracle.e4m3_value(byte)
        if byte in (0x7F, 0xFF):
            assert math.isnan(v) and math.isnan(ref[byte])
        else:
            assert v == ref[byte], hex(byte)


def test_e4m3_spot_values():
    assert oracle.e4m3_value(0x38) == 1.0
    assert oracle.e4m3_value(0x30) == 0.5
    assert oracle.e4m3_value(0x40) == 2.0
    assert oracle.e4m3_value(0x4C) == 6.0
    assert oracle.e4m3_value(0x7E) == 448.0
    assert oracle.e4m3_value(0x01) == 2.0 ** -9
    assert oracle.e4m3_value(0x08) == 2.0 ** -6
    assert oracle.e4m3_value(0x80) == 0.0 and math.copysign(1, oracle.e4m3_value(0x80)) < 0


# ---- P3: encoders vs exact-rational brute force ---------------------------------------------
def brute_nearest_even(a, b, values):
    """Index of the value nearest the exact rational a/b, ties to the even index.

    Independent of the oracle: every distance is an exact Fraction and all
    candidates are compared; saturation falls out because the largest value is
    nearest to anything above it.
    """
    r = Fraction(a) / Fraction(b)
    best, best_d = None, None
    for k, v in enumerate(values):
        d = abs(r - Fraction(v))
        if best is None or d < best_d or (d == best_d and k % 2 == 0):
            best, best_d = k, d
    return best


E4M3_POS = torch_e4m3_values()[:127]          # codes 0x00..0x7E from torch, increasing
assert all(E4M3_POS[i] < E4M3_POS[i + 1] for i in range(126))


def bf16_round(x: float) -> float:
    return torch.tensor(x, dtype=torch.float32).to(torch.bfloat16).item()


def fp32_round(x: float) -> float:
    return float(np.float32(x))


def e4m3_cases(rng):
    cases = []
    for _ in range(400):                                   # random group maxima and scales
        a = bf16_round(abs(rng.gauss(0, 1)) * 10 ** rng.uniform(-4, 4))
        g = fp32_round(10 ** rng.uniform(-6, 2))
        cases.append((a, 6.0 * g))
    for k in range(126):                                   # every midpoint, exactly and +-1 ulp
        mid = (E4M3_POS[k] + E4M3_POS[k + 1]) / 2
        g = fp32_round(rng.uniform(0.001, 4.0))
        b = 6.0 * g
        a = mid * b                                        # exact: <= 31 significant bits
        cases += [(a, b), (math.nextafter(a, math.inf), b), (math.nextafter(a, 0.0), b)]
    cases += [(0.0, 1.0), (500.0, 1.0), (448.0 * 6, 6.0), (2.0 ** -10, 1.0), (3 * 2.0 ** -10, 1.0),
              (1.0625, 1.0), (1.1875, 1.0), (1e30, 1.0)]
    return cases


def test_e4m3_encode_matches_bruteforce():
    rng = random.Random(1234)
    for a, b in e4m3_cases(rng):
        assert oracle.e4m3_encode(a, b) == brute_nearest_even(a, b, E4M3_POS), (a, b)


def test_e4m3_encode_tie_examples():
    assert oracle.e4m3_encode(1.0625, 1.0) == 0x38       # 1.0625 -> 1.0
    assert oracle.e4m3_encode(1.1875, 1.0) == 0x3A       # 1.1875 -> 1.25
    assert oracle.e4m3_encode(2.0 ** -10, 1.0) == 0x00   # 2^-10 -> 0
    assert oracle.e4m3_encode(3 * 2.0 ** -10, 1.0) == 0x02  # -> 2^-8
    assert oracle.e4m3_encode(500.0, 1.0) == 0x7E        # saturates at 448
    assert oracle.e4m3_encode(1.0, 0.0) == 0x00


def test_e4m3_encode_matches_torch_rounding():
    """torch rounds fp32 to float8_e4m3fn to nearest, ties to even (a library routine)."""
    rng = np.random.default_rng(7)
    x = np.concatenate([rng.uniform(0, 448, 3000), 2.0 ** rng.uniform(-12, 8.8, 3000)]).astype(np.float32)
    x = x[x <= 448]
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v), 1.0) for v in x])
    assert np.array_equal(got, ref)


def test_e2m1_encode_matches_bruteforce():
    rng = random.Random(99)
    mags = E2M1_BY_CODE
    cases = []
    for _ in range(2000):
        b = fp32_round(10 ** rng.uniform(-5, 3)) * E4M3_POS[rng.randrange(1, 127)]
        a = bf16_round(abs(rng.gauss(0, 3)) * b)
        cases.append((a, b))
    for k in range(7):
        mid = (mags[k] + mags[k + 1]) / 2
        for s in (1, 448, 2.0 ** -9, 0.875):
            for g in (1.0, fp32_round(1 / 2688), fp32_round(3.7)):
                b = s * g
                a = mid * b
                cases += [(a, b), (math.nextafter(a, math.inf), b), (math.nextafter(a, 0.0), b)]
    cases += [(0.0, 1.0), (100.0, 1.0), (6.0, 1.0), (5.0, 1.0)]
    for a, b in cases:
        assert oracle.e2m1_encode(a, b) == brute_nearest_even(a, b, mags), (a, b)
    assert oracle.e2m1_encode(1.0, 0.0) == 0


# ---- global scale -------------------------------------------------------------------------
def test_global_scale_is_nearest_fp32_of_amax_over_2688():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 300))
        x = (rng.standard_normal(n) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32)
        xb = torch.from_numpy(x).to(torch.bfloat16)
        u16 = xb.view(torch.int16).numpy().view(np.uint16)
        g = oracle.global_scale(u16)
        amax = Fraction(float(xb.abs().max().item()))
        exact = amax / 2688
        gf = np.float32(g)
        d = abs(Fraction(float(gf)) - exact)
        for nb in (np.nextafter(gf, np.float32(np.inf)), np.nextafter(gf, np.float32(0))):
            dn = abs(Fraction(float(nb)) - exact)
            assert d < dn or (d == dn and (gf.view(np.uint32) & 1) == 0)
    z = np.zeros(5, dtype=np.uint16)
    assert oracle.global_scale(z) == 0.0
    assert oracle.global_scale(np.array([0x4528], dtype=np.uint16)) == 1.0   # bf16 2688 -> g = 1


# ---- hand-worked golden rows ------------------------------------------------------------
def _golden_rows():
    spec = json.load(open(GOLDEN))
    D = spec["head_dim"]
    rows = []
    base = spec["rows"][0]
    x0 = [v for grp in base["groups"] for v in grp["x"]]
    sc0 = [grp["scale"] for grp in base["groups"]]
    cd0 = [c for grp in base["groups"] for c in grp["codes"]]
    rows.append((x0, base["g"], sc0, cd0))
    for r in spec["rows"][1:]:
        assert r["same_as_row"] == 0
        rows.append(([v * r["x_scale"] for v in x0], r["g"], sc0, cd0))
    return D, rows


def test_quantizer_hand_worked_rows():
    D, rows = _golden_rows()
    for x, g, scales, codes in rows:
        assert len(x) == D
        xb = torch.tensor(x, dtype=torch.float32).to(torch.bfloat16)
        assert xb.to(torch.float32).tolist() == [float(v) for v in x]        # inputs exact in bf16
        u16 = xb.view(torch.int16).numpy().view(np.uint16).reshape(1, D)
        c, s = oracle.quantize_rows(u16, np.float32(g))
        assert s.reshape(-1).tolist() == scales
        assert c.reshape(-1).tolist() == codes


# ---- P4: size arithmetic ------------------------------------------------------------------
def test_packed_size_arithmetic():
    import workloads
    for D in (128, 256):
        per_elem = (D // 2 + D // 16) / D                 # codes + one E4M3 byte per 16
        assert per_elem == 0.5625
        assert workloads.packed_bytes_per_token_head(D) == 2 * D * 0.5625
    # int8 with one 2-byte scale per group of 64 (1.03125 B/element) vs NVFP4:
    saving = 1 - 0.5625 / (1 + 2 / 64)
    assert abs(saving - 0.4545) < 1e-3                   # the pages' "45% less KV VRAM than int8"
    assert 1 - 0.5625 / 1.0 == 0.4375                    # vs bare int8
    c = oracle.Cache(4, 256, 1000)
    planes = c.k_codes.nbytes + c.k_scales.nbytes + c.v_codes.nbytes + c.v_scales.nbytes
    assert planes == 1000 * 4 * 2 * (256 // 2 + 256 // 16)
