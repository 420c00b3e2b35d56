"""NVFP4-KV CPU oracle (fp64) -- test infrastructure only.

Only ``tests/``, the smoke check in ``__graft_entry__`` and the CPU-baseline leg
of ``bench.py`` may import this package. The product path (the HIP library and
its Python binding) never imports it, and this package imports nothing of the
product path: the two share no code.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, fp64, built by gcc without
fast-math and without FMA contraction); this module is argument marshalling.

What each function follows (gzenz/ninfer page, section "Context and model",
bullet "NVFP4 KV cache": 4-bit E2M1 codes with E4M3 group-16 scales) and the
readings where the pages are silent are stated in the C file's header.

Pins (tests run with ``-m "not gpu"``):
  * e2m1_value / e4m3_value: closed forms of the OCP MX v1.0 formats, all codes;
    E4M3 also against torch.float8_e4m3fn decoding.
  * e2m1_encode / e4m3_encode: exact-rational brute-force nearest search with
    ties to even; E4M3 also against torch's float8_e4m3fn rounding.
  * global_scale: the nearest fp32 to amax/2688, checked with exact rationals.
  * quantize_rows: hand-worked groups under tests/golden (ties, saturation,
    subnormal scales, signed zero, nibble order) and the error-bound invariants.
  * dequantize_rows: the quantiser's error bound against the original inputs.
  * attention: torch float64 scaled_dot_product_attention on the dequantised
    tensors, brute-force invariants and the causal reduction.
  * quantize_rows_fp8 / dequantize_rows_fp8 (the K half of K8V4, row-scaled FP8
    E4M3): hand-worked rows under tests/golden, exact-rational brute force of the
    row scale and every code, error-bound and re-encoding invariants.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_nvfp4.so")
_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, fp64, no fast-math, no FMA contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math", "-ffp-contract=off",
               "-pthread", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        build()
        lib = ctypes.CDLL(_LIB)
        c_i32, c_i64, c_dbl, c_f32, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_double, ctypes.c_float, ctypes.c_void_p
        lib.orc_e2m1_value.argtypes = [ctypes.c_int]
        lib.orc_e2m1_value.restype = c_dbl
        lib.orc_e4m3_value.argtypes = [ctypes.c_int]
        lib.orc_e4m3_value.restype = c_dbl
        lib.orc_e4m3_encode.argtypes = [c_dbl, c_dbl]
        lib.orc_e4m3_encode.restype = ctypes.c_int
        lib.orc_e2m1_encode.argtypes = [c_dbl, c_dbl]
        lib.orc_e2m1_encode.restype = ctypes.c_int
        lib.orc_global_scale.argtypes = [vp, c_i64]
        lib.orc_global_scale.restype = c_f32
        lib.orc_quantize_rows.argtypes = [vp, c_i64, c_i32, vp, vp, vp, ctypes.c_int]
        lib.orc_quantize_rows.restype = None
        lib.orc_dequantize_rows.argtypes = [vp, vp, c_i64, c_i32, vp, vp]
        lib.orc_dequantize_rows.restype = None
        lib.orc_quantize_rows_fp8.argtypes = [vp, c_i64, c_i32, vp, vp, ctypes.c_int]
        lib.orc_quantize_rows_fp8.restype = None
        lib.orc_dequantize_rows_fp8.argtypes = [vp, vp, c_i64, c_i32, vp]
        lib.orc_dequantize_rows_fp8.restype = None
        lib.orc_attention.argtypes = [vp, vp, vp, vp, c_i32, c_i32, c_i32, c_i64, vp, vp, c_i32, vp, vp,
                                      c_i32, c_i32, c_dbl, c_i64, vp, vp, ctypes.c_int]
        lib.orc_attention.restype = ctypes.c_int
        _lib = lib
        return lib


def default_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


# ---- formats ------------------------------------------------------------------
def e2m1_value(code: int) -> float:
    return _load().orc_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().orc_e4m3_value(int(byte))


def e4m3_encode(a: float, b: float) -> int:
    """E4M3 code (0..0x7E) nearest the real a/b, ties to even, saturating at 448."""
    return _load().orc_e4m3_encode(float(a), float(b))


def e2m1_encode(a: float, b: float) -> int:
    """E2M1 magnitude code (0..7) nearest the real a/b, ties to even, saturating at 6."""
    return _load().orc_e2m1_encode(float(a), float(b))


# ---- quantiser ------------------------------------------------------------------
def global_scale(x_u16: np.ndarray) -> np.float32:
    """fp32(amax / 2688) over bf16 bit patterns."""
    x = np.ascontiguousarray(x_u16, dtype=np.uint16)
    return np.float32(_load().orc_global_scale(_ptr(x), x.size))


def calibrate(k_rows: np.ndarray, v_rows: np.ndarray, seq_lens) -> np.ndarray:
    """g[b][h][0|1] for rows bf16 [sum L][Hkv][D] concatenated over sequences."""
    B = len(seq_lens)
    Hkv = k_rows.shape[1]
    g = np.zeros((B, Hkv, 2), dtype=np.float32)
    base = 0
    for b, L in enumerate(seq_lens):
        for h in range(Hkv):
            g[b, h, 0] = global_scale(np.ascontiguousarray(k_rows[base:base + L, h]))
            g[b, h, 1] = global_scale(np.ascontiguousarray(v_rows[base:base + L, h]))
        base += L
    return g


def quantize_rows(x_u16: np.ndarray, g, nthreads: int | None = None):
    """Quantise rows [..., D] of bf16 bit patterns; g is a scalar or one fp32 per row.

    Returns (codes uint8 [..., D/2], scales uint8 [..., D/16]).
    """
    x = np.ascontiguousarray(x_u16, dtype=np.uint16)
    D = x.shape[-1]
    assert D % 16 == 0
    n = x.size // D
    gv = np.ascontiguousarray(np.broadcast_to(np.asarray(g, dtype=np.float32).reshape(-1), (n,))
                              if np.asarray(g).size == 1 else np.asarray(g, dtype=np.float32).reshape(n))
    codes = np.empty(x.shape[:-1] + (D // 2,), dtype=np.uint8)
    scales = np.empty(x.shape[:-1] + (D // 16,), dtype=np.uint8)
    _load().orc_quantize_rows(_ptr(x), n, D, _ptr(gv), _ptr(codes), _ptr(scales),
                              nthreads or default_threads())
    return codes, scales


def dequantize_rows(codes: np.ndarray, scales: np.ndarray, g) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.uint8)
    D = c.shape[-1] * 2
    n = c.size // (D // 2)
    gv = np.ascontiguousarray(np.broadcast_to(np.asarray(g, dtype=np.float32).reshape(-1), (n,))
                              if np.asarray(g).size == 1 else np.asarray(g, dtype=np.float32).reshape(n))
    out = np.empty(c.shape[:-1] + (D,), dtype=np.float64)
    _load().orc_dequantize_rows(_ptr(c), _ptr(s), n, D, _ptr(gv), _ptr(out))
    return out


def quantize_rows_fp8(x_u16: np.ndarray, nthreads: int | None = None):
    """Row-scaled FP8 E4M3 (the K half of K8V4) of rows [..., D] of bf16 bit patterns.

    Returns (codes uint8 [..., D], scales float32 [...]): s = fp32(amax_row / 448), code =
    sign << 7 | nearest E4M3 magnitude code of |x| / s (ties to even, saturating at 448).
    """
    x = np.ascontiguousarray(x_u16, dtype=np.uint16)
    D = x.shape[-1]
    n = x.size // D
    codes = np.empty(x.shape, dtype=np.uint8)
    scales = np.empty(x.shape[:-1], dtype=np.float32)
    _load().orc_quantize_rows_fp8(_ptr(x), n, D, _ptr(codes), _ptr(scales), nthreads or default_threads())
    return codes, scales


def dequantize_rows_fp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    s = np.ascontiguousarray(scales, dtype=np.float32)
    D = c.shape[-1]
    out = np.empty(c.shape, dtype=np.float64)
    _load().orc_dequantize_rows_fp8(_ptr(c), _ptr(s), c.size // D, D, _ptr(out))
    return out


KV_FORMATS = ("nvfp4", "k8v4")


class Cache:
    """Host copy of the packed KV pool.

    nvfp4: K and V planes [Hkv][capacity][D/2] codes and [Hkv][capacity][D/16] E4M3 scales.
    k8v4:  V as above; K codes [Hkv][capacity][D] (E4M3) and fp32 row scales [Hkv][capacity].
    """

    def __init__(self, num_kv_heads: int, head_dim: int, capacity: int, kv_format: str = "nvfp4"):
        assert kv_format in KV_FORMATS
        self.Hkv, self.D, self.capacity, self.kv_format = num_kv_heads, head_dim, capacity, kv_format
        self.v_codes = np.zeros((num_kv_heads, capacity, head_dim // 2), dtype=np.uint8)
        self.v_scales = np.zeros((num_kv_heads, capacity, head_dim // 16), dtype=np.uint8)
        if kv_format == "k8v4":
            self.k_codes = np.zeros((num_kv_heads, capacity, head_dim), dtype=np.uint8)
            self.k_scales = np.zeros((num_kv_heads, capacity), dtype=np.float32)
        else:
            self.k_codes = np.zeros_like(self.v_codes)
            self.k_scales = np.zeros_like(self.v_scales)


def append(cache: Cache, k_new: np.ndarray, v_new: np.ndarray, g: np.ndarray, seq_base, write_pos,
           n_new, nthreads: int | None = None) -> None:
    """Quantise n_new[b] rows per sequence (bf16 [sum n_new][Hkv][D], concatenated over b)
    into slots seq_base[b] + write_pos[b] + r of every head plane, with g[b][h][0|1] (K8V4:
    K rows row-scaled FP8, g[b][h][0] unused)."""
    r0 = 0
    for b, n in enumerate(n_new):
        if n == 0:
            continue
        s0 = seq_base[b] + write_pos[b]
        assert s0 + n <= cache.capacity
        for h in range(cache.Hkv):
            if cache.kv_format == "k8v4":
                kc, ks = quantize_rows_fp8(k_new[r0:r0 + n, h], nthreads)
            else:
                kc, ks = quantize_rows(k_new[r0:r0 + n, h], g[b, h, 0], nthreads)
            vc, vs = quantize_rows(v_new[r0:r0 + n, h], g[b, h, 1], nthreads)
            cache.k_codes[h, s0:s0 + n] = kc
            cache.k_scales[h, s0:s0 + n] = ks
            cache.v_codes[h, s0:s0 + n] = vc
            cache.v_scales[h, s0:s0 + n] = vs
        r0 += n


def attention(cache: Cache, g: np.ndarray, q_u16: np.ndarray, seq_base, seq_len, n_q: int,
              sm_scale: float, sel=None, nthreads: int | None = None) -> np.ndarray:
    """fp64 decode attention. q is bf16 bits [B][n_q][Hq][D].

    sel: iterable of (b, i, h); default all. Returns float64 [len(sel)][D], or
    [B][n_q][Hq][D] when sel is None.
    """
    q = np.ascontiguousarray(q_u16, dtype=np.uint16)
    B, nq, Hq, D = q.shape
    assert nq == n_q and D == cache.D
    full = sel is None
    if full:
        sel = [(b, i, h) for b in range(B) for i in range(n_q) for h in range(Hq)]
    sel_a = np.ascontiguousarray(np.asarray(sel, dtype=np.int32).reshape(-1, 3))
    out = np.empty((sel_a.shape[0], D), dtype=np.float64)
    gs = np.ascontiguousarray(g, dtype=np.float32)
    base = np.ascontiguousarray(seq_base, dtype=np.int64)
    lens = np.ascontiguousarray(seq_len, dtype=np.int64)
    rc = _load().orc_attention(_ptr(cache.k_codes), _ptr(cache.k_scales), _ptr(cache.v_codes),
                               _ptr(cache.v_scales), 1 if cache.kv_format == "k8v4" else 0, cache.Hkv, D,
                               cache.capacity, _ptr(gs), _ptr(q), B,
                               _ptr(base), _ptr(lens), n_q, Hq, float(sm_scale), sel_a.shape[0],
                               _ptr(sel_a), _ptr(out), nthreads or default_threads())
    if rc != 0:
        raise ValueError("oracle attention: invalid arguments")
    return out.reshape(B, n_q, Hq, D) if full else out
