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
