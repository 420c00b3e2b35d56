"""The device group quantiser, built for the host, against the oracle (no GPU needed).

quantize.h decides every rounding with integer and fp32/fp64 arithmetic that is the same on
the host; the host build (tests/host/quantize_host.cpp) replaces only v_perm_b32 and the
fp64 reciprocal. The reciprocal is perturbed by up to 2^-12 relative, so the exact
correction of the approximate scale code is exercised. Cases: every positive bf16 value as a
group maximum, groups at every E4M3 midpoint (x 6 g) and every E2M1 midpoint (x S g) with
their bf16 neighbours under random and extreme global scales, random groups and scales, and
the adversarial groups of the GPU test.
"""
import ctypes
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from helpers import adversarial_rows

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "quantized_kv_decode_amd", "csrc")
CLANG = "/opt/rocm/llvm/bin/clang++"


run_fp8_holder = []


@pytest.fixture(scope="module")
def host_quantizer(tmp_path_factory):
    cxx = CLANG if os.path.exists(CLANG) else shutil.which("clang++")
    if cxx is None:
        pytest.skip("no clang++ for the host build of the device quantiser")
    out = str(tmp_path_factory.mktemp("hostq") / "libquantize_host.so")
    subprocess.run([cxx, "-O2", "-std=c++17", "-fPIC", "-shared", "-I", os.path.join(HERE, "host"), "-I", CSRC,
                    os.path.join(HERE, "host", "quantize_host.cpp"), "-o", out], check=True)
    lib = ctypes.CDLL(out)
    lib.quantize_groups.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_void_p, ctypes.c_void_p,
                                    ctypes.c_void_p, ctypes.c_double]

    lib.quantize_rows_fp8.argtypes = [ctypes.c_void_p, ctypes.c_long, ctypes.c_int, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_double]

    def run_fp8(x, eps):
        x = np.ascontiguousarray(x, np.uint16)
        n, D = x.shape
        codes = np.zeros((n, D), np.uint8)
        scales = np.zeros(n, np.float32)
        lib.quantize_rows_fp8(x.ctypes.data, n, D, codes.ctypes.data, scales.ctypes.data, eps)
        return codes, scales
    run_fp8_holder.append(run_fp8)

    def run(x, g, eps):
        x = np.ascontiguousarray(x, np.uint16)
        g = np.ascontiguousarray(g, np.float32)
        n = x.shape[0]
        codes = np.zeros((n, 8), np.uint8)
        scales = np.zeros(n, np.uint8)
        lib.quantize_groups(x.ctypes.data, n, g.ctypes.data, codes.ctypes.data, scales.ctypes.data, eps)
        return codes, scales
    return run


def check(run, x, g):
    rc, rs = oracle.quantize_rows(x, g)
    rc, rs = rc.reshape(-1, 8), rs.reshape(-1)
    for eps in (0.0, 2.0 ** -20, -2.0 ** -20, 2.0 ** -12, -2.0 ** -12):
        c, s = run(x, g, eps)
        bad = np.nonzero((c != rc).any(1) | (s != rs))[0]
        assert bad.size == 0, (f"eps {eps}: {bad.size} groups differ, first {bad[0]}: g {g[bad[0]]} x {x[bad[0]]} "
                               f"scale {s[bad[0]]} vs {rs[bad[0]]}")


@pytest.mark.parametrize("gval", [1.0, 0.5, 3.0, 0.0, 1e-30, 7.1e-36, 1e-40, 2.5e30, 3.0e38, 1.4e-45])
def test_adversarial_groups(host_quantizer, gval):
    x = adversarial_rows(256).reshape(-1, 16)
    check(host_quantizer, x, np.full(x.shape[0], gval, np.float32))


@pytest.mark.parametrize("gval", [1.0, 1 / 2688, 0.37, 1e-20, 1e-41, 1e30])
def test_every_bf16_value_as_group_max(host_quantizer, gval):
    rng = np.random.default_rng(1)
    top = np.arange(0, 0x7F80, dtype=np.uint16)
    x = np.zeros((top.size, 16), np.uint16)
    x[:, 0] = top
    x[:, 1:] = np.minimum(rng.integers(0, 0x8000, (top.size, 15)), top[:, None]).astype(np.uint16)
    x[:, 1:] |= (rng.integers(0, 2, (top.size, 15)) << 15).astype(np.uint16)
    check(host_quantizer, x, np.full(top.size, gval, np.float32))


def test_random_groups_and_scales(host_quantizer):
    rng = np.random.default_rng(2)
    n = 20000
    g = (rng.random(n) * 2.0 ** rng.integers(-140, 120, n)).astype(np.float32)
    check(host_quantizer, rng.integers(0, 0x7F80, (n, 16)).astype(np.uint16), g)


def test_groups_on_midpoints(host_quantizer):
    """Group maxima on E4M3 midpoints x 6 g and elements on E2M1 midpoints x S g (or one bf16
    ulp above), with g a small integer times a power of two, so that ties are exact."""
    rng = np.random.default_rng(3)
    n = 30000
    g = (2.0 ** rng.integers(-140, 100, n) * rng.integers(1, 9, n)).astype(np.float32)
    e4 = np.array([oracle.e4m3_value(c) for c in range(127)])
    k = rng.integers(0, 126, n)

    def bf16_down(v):
        return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)

    x = np.zeros((n, 16), np.uint16)
    x[:, 0] = (bf16_down(0.5 * (e4[k] + e4[k + 1]) * 6 * g.astype(np.float64)) + rng.integers(0, 2, n)) & 0x7FFF
    Sg = e4[np.clip(k + rng.integers(0, 2, n), 0, 126)] * g
    for j in range(1, 16):
        t = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])[rng.integers(0, 7, n)]
        x[:, j] = (bf16_down(t * Sg) + rng.integers(0, 2, n)) & 0x7FFF
        x[:, j] |= (rng.integers(0, 2, n) << 15).astype(np.uint16)
    check(host_quantizer, x, g)


# ---- row-scaled FP8 E4M3 (K8V4's K rows) ---------------------------------------------------
def check_fp8(x):
    rc, rs = oracle.quantize_rows_fp8(x)
    for eps in (0.0, 2.0 ** -20, -2.0 ** -20, 2.0 ** -12, -2.0 ** -12):
        c, s = run_fp8_holder[0](x, eps)
        assert np.array_equal(s.view(np.uint32), rs.view(np.uint32)), f"eps {eps}: row scales differ"
        bad = np.nonzero((c != rc).any(1))[0]
        assert bad.size == 0, f"eps {eps}: {bad.size} rows differ, first {bad[0]}"


def test_fp8_rows_every_bf16_value_as_row_max(host_quantizer):
    """Every positive finite bf16 value as a row's maximum (so every row scale that can occur),
    with the row's other elements at fixed fractions of it that straddle E4M3 midpoints."""
    mags = np.arange(1, 0x7F80, dtype=np.uint32)
    D = 128
    x = np.zeros((mags.size, D), np.uint16)
    x[:, 0] = mags
    f = np.frombuffer((mags << 16).astype(np.uint32).tobytes(), np.float32).astype(np.float64)
    fr = [0.999, 0.5, 0.4375, 0.1, 1 / 3, 2.0 ** -7, 0.0023, 0.03125 * 1.0625, 3 * 2.0 ** -19, 0.77]
    for k, t in enumerate(fr):
        v = (f * t).astype(np.float32)
        b = (np.frombuffer(v.tobytes(), np.uint32) >> 16).astype(np.uint16)   # truncated to bf16
        x[:, 1 + k] = b | (0x8000 if k % 2 else 0)
    check_fp8(x)


def test_fp8_rows_on_midpoints(host_quantizer):
    """Rows whose scale is a power of two (amax = 448 * 2^k) and whose elements sit on every E4M3
    midpoint and one bf16 step either side of it."""
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    rows = []
    for k in (-20, -6, 0, 5, 17):
        mids = np.array([(e4[i] + e4[i + 1]) / 2 * 2.0 ** k for i in range(126)], np.float32)
        mb = (np.frombuffer(mids.tobytes(), np.uint32) >> 16).astype(np.uint16)
        vals = np.concatenate([mb, mb + 1, mb - 1]).astype(np.uint16)
        for i in range(0, vals.size, 255):
            row = np.zeros(256, np.uint16)
            top = np.array([448 * 2.0 ** k], np.float32)
            row[0] = (np.frombuffer(top.tobytes(), np.uint32) >> 16)[0]
            chunk = vals[i:i + 255]
            row[1:1 + chunk.size] = chunk
            rows.append(row)
    check_fp8(np.stack(rows))


def test_fp8_rows_around_the_fp32_path_threshold(host_quantizer):
    """Row scales just above and below 2^-60 (the fp32 and the fp64 decision paths), with
    elements on E4M3 midpoints of their scale and one bf16 step either side."""
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    rows = []
    for k in (-61, -60, -59):
        for f in (0.999, 1.0, 1.001):
            top = np.array([448 * 2.0 ** k * f], np.float32)
            tb = (np.frombuffer(top.tobytes(), np.uint32) >> 16)[0]
            s = float(np.float32(float(bf16_value(tb)) / 448))
            mids = np.array([(e4[i] + e4[i + 1]) / 2 * s for i in range(126)], np.float32)
            mb = (np.frombuffer(mids.tobytes(), np.uint32) >> 16).astype(np.uint16)
            vals = np.concatenate([mb, mb + 1, mb - 1]).astype(np.uint16)
            for i in range(0, vals.size, 255):
                row = np.zeros(256, np.uint16)
                row[0] = tb
                chunk = vals[i:i + 255]
                row[1:1 + chunk.size] = chunk
                rows.append(row)
    check_fp8(np.stack(rows))


def bf16_value(bits):
    return np.frombuffer((np.uint32(bits) << np.uint32(16)).tobytes(), np.float32)[0]


def test_fp8_rows_random_and_edge(host_quantizer):
    rng = np.random.default_rng(17)
    x = (rng.standard_normal((500, 256)) * 10.0 ** rng.uniform(-30, 30, (500, 1))).astype(np.float32)
    xb = (np.frombuffer(x.tobytes(), np.uint32) >> 16).astype(np.uint16).reshape(500, 256)
    edge = np.zeros((4, 256), np.uint16)
    edge[1, :] = 0x8000                                        # all -0
    edge[2, 5] = 0x0001                                        # smallest bf16 subnormal as the max
    edge[3, 7] = 0x7F7F                                        # largest finite bf16
    check_fp8(np.concatenate([xb, edge]))


def test_calibrated_scales_near_ties(host_quantizer):
    """Groups and rows under scales calibrated from their own data -- g = fp32(amax / 2688), row
    scale fp32(amax / 448), amax a bf16 value -- for every amax significand of a binade. With
    8-bit significands, many quotients then lie within 2^-24 of an E2M1 or E4M3 midpoint (the
    rounding of the scale decides them): the regime in which the fast path's hardware bounds
    round apart and its exact midpoint test decides."""
    rng = np.random.default_rng(5)
    amax = (0x4000 + np.arange(128)).astype(np.uint16)            # 2.0 .. 3.98, every significand
    av = np.array([bf16_value(a) for a in amax], np.float64)
    n = 96
    x = np.zeros((amax.size, n, 16), np.uint16)
    for i, a in enumerate(amax):
        v = (rng.uniform(0, 1, (n, 16)) * av[i]).astype(np.float32)
        b = (np.frombuffer(v.tobytes(), np.uint32) >> 16).astype(np.uint16).reshape(n, 16)
        b |= (rng.integers(0, 2, (n, 16)) << 15).astype(np.uint16)
        b[:, 0] = a                                                # the sequence maximum in every group
        x[i] = b
    g = np.repeat(np.array([np.float32(v / 2688) for v in av], np.float32), n)
    check(host_quantizer, x.reshape(-1, 16), g)
    check_fp8(x.reshape(-1, 256))


def test_fast_path_range_edges(host_quantizer):
    """Global scales at the edges of the fast path's range (2^-100 and 2^100, exactly and one
    ulp either side) and FP8 row scales around 2^-100 (rows with amax near 448 * 2^-100) and
    near the largest bf16: groups on either side of the switch between the hardware-conversion
    path and the exact decision agree with the oracle."""
    ulp = lambda v, k: np.array([np.nextafter(np.float32(v), np.float32(np.inf if k > 0 else 0))], np.float32)[0]
    gs = []
    for e in (-100, 100):
        v = np.float32(2.0 ** e)
        gs += [v, ulp(v, 1), ulp(v, -1)]
    x = adversarial_rows(256).reshape(-1, 16)
    rng = np.random.default_rng(9)
    rnd = rng.integers(0, 0x7F80, (400, 16)).astype(np.uint16)
    for gv in gs:
        check(host_quantizer, x, np.full(x.shape[0], gv, np.float32))
        check(host_quantizer, rnd, np.full(rnd.shape[0], gv, np.float32))
    # FP8 rows: maxima 448 * 2^-100 and its bf16 neighbours (row scales around 2^-100), and
    # the largest finite bf16 magnitudes
    tops = []
    t = np.array([448 * 2.0 ** -100], np.float32)
    tb = int((np.frombuffer(t.tobytes(), np.uint32) >> 16)[0])
    tops += [tb - 1, tb, tb + 1, 0x7F7F, 0x7F7E]
    rows = np.zeros((len(tops) * 4, 128), np.uint16)
    for i, top in enumerate(tops):
        for r in range(4):
            row = rng.integers(0, top + 1, 128).astype(np.uint16)
            row[0] = top
            row |= (rng.integers(0, 2, 128) << 15).astype(np.uint16) * (np.arange(128) > 0)
            rows[4 * i + r] = row
    check_fp8(rows)
