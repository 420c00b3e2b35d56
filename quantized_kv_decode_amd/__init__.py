"""MI355X (gfx950) NVFP4-KV decode attention: Python binding of libnvfp4kv.so.

Argument marshalling only. Every step of the path (calibration, quantise-on-
append, split-K decode, combine) runs in the HIP kernels behind the C ABI in
include/nvfp4_kv.h; PyTorch supplies device memory and the current stream.
If the library has not been built this module raises on first use (there is no
fallback implementation).

The method: K/V stored as 4-bit E2M1 codes with E4M3 group-16 scales (gzenz/ninfer
page, "Context and model", NVFP4 KV cache bullet), read directly by grouped-query
decode attention with 1 + draft query tokens (knoopx/ninfer page, "Capabilities
and limits").
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4kv.so")

OK, EINVAL, EUNSUPPORTED, ERANGE, EWORKSPACE, EHIP = 0, -1, -2, -3, -4, -5
OUT_F32, OUT_BF16 = 0, 1
MAX_SEQS, MAX_ROWS = 8, 8192

_ERR_NAMES = {EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", ERANGE: "ERANGE",
              EWORKSPACE: "EWORKSPACE", EHIP: "EHIP"}

SYMBOLS = ["nvfp4_kv_calibrate", "nvfp4_kv_append", "nvfp4_decode_attn_workspace_bytes",
           "nvfp4_decode_attn", "nvfp4_decode_step", "nvfp4_decode_step_dev_len", "nvfp4_decode_step_noalloc",
           "nvfp4_decode_attn_partial", "nvfp4_decode_attn_combine", "nvfp4_hbm_read_probe",
           "nvfp4_last_error"]


class Nvfp4Error(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{_ERR_NAMES.get(code, code)}: {msg}")
        self.code = code


KV_NVFP4, KV_K8V4 = 0, 1
KV_FORMATS = {"nvfp4": KV_NVFP4, "k8v4": KV_K8V4}


class CacheDesc(ctypes.Structure):
    _fields_ = [("k_codes", ctypes.c_void_p), ("k_scales", ctypes.c_void_p),
                ("v_codes", ctypes.c_void_p), ("v_scales", ctypes.c_void_p),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("kv_format", ctypes.c_int32)]


_lib = None


def load_library():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m quantized_kv_decode_amd.build` "
                           "(or __graft_entry__.build()); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64), ctypes.c_float, ctypes.c_size_t
    P = ctypes.POINTER(CacheDesc)
    lib.nvfp4_kv_calibrate.argtypes = [P, vp, vp, i32, i64, vp, vp]
    lib.nvfp4_kv_append.argtypes = [P, vp, vp, vp, i32, i64, i64, i64, vp]
    lib.nvfp4_decode_attn_workspace_bytes.argtypes = [P, i32, i64, i32, i32]
    lib.nvfp4_decode_attn_workspace_bytes.restype = sz
    lib.nvfp4_decode_attn.argtypes = [P, vp, vp, vp, i32, i32, i64, i64, i32, i32, f32, vp, sz, vp]
    lib.nvfp4_decode_step.argtypes = [P, vp, vp, vp, vp, vp, i32, i32, i64, i64, i32, i32, f32, vp, sz, vp]
    lib.nvfp4_decode_step_dev_len.argtypes = [P, vp, vp, vp, vp, vp, i32, i32, i64, i64, vp, i32, i32, f32, vp, sz,
                                              vp]
    lib.nvfp4_decode_attn_partial.argtypes = [P, vp, vp, i32, i64, i64, i32, i32, f32, vp, sz, vp]
    lib.nvfp4_decode_attn_combine.argtypes = [P, vp, vp, i32, i32, i64, i32, i32, vp, sz, vp]
    lib.nvfp4_hbm_read_probe.argtypes = [vp, sz, vp, i32, vp]
    lib.nvfp4_decode_step_noalloc.argtypes = [P, vp, vp, vp, vp, vp, i32, i32, i64, i64, i32, i32, f32, vp]
    lib.nvfp4_last_error.argtypes = []
    lib.nvfp4_last_error.restype = ctypes.c_char_p
    for f in ("nvfp4_kv_calibrate", "nvfp4_kv_append", "nvfp4_decode_attn", "nvfp4_decode_step",
              "nvfp4_decode_step_dev_len", "nvfp4_decode_attn_partial", "nvfp4_decode_attn_combine",
              "nvfp4_hbm_read_probe", "nvfp4_decode_step_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int) -> None:
    if rc != OK:
        raise Nvfp4Error(rc, load_library().nvfp4_last_error().decode())


def _i64(values):
    vals = [int(v) for v in values]
    arr = (ctypes.c_int64 * max(1, len(vals)))(*vals)
    return ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))


def _stream(stream=None) -> int:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _ptr(t) -> int:
    return 0 if t is None else t.data_ptr()


class KVPool:
    """Caller-owned pool: code and scale planes for K and V (torch tensors on the device).

    nvfp4: every plane uint8, codes [Hkv][capacity][D/2], scales [Hkv][capacity][D/16].
    k8v4:  V as above; K codes uint8 [Hkv][capacity][D] (E4M3), K row scales float32 [Hkv][capacity].
    """

    def __init__(self, num_kv_heads: int, head_dim: int, capacity: int, device="cuda", kv_format: str = "nvfp4"):
        self.num_kv_heads, self.head_dim, self.capacity = num_kv_heads, head_dim, capacity
        self.kv_format = kv_format
        mk = lambda w: torch.zeros((num_kv_heads, capacity, w), dtype=torch.uint8, device=device)
        if kv_format == "k8v4":
            self.k_codes = mk(head_dim)
            self.k_scales = torch.zeros((num_kv_heads, capacity), dtype=torch.float32, device=device)
        elif kv_format == "nvfp4":
            self.k_codes, self.k_scales = mk(head_dim // 2), mk(head_dim // 16)
        else:
            raise ValueError(f"kv_format {kv_format!r}: 'nvfp4' or 'k8v4'")
        self.v_codes, self.v_scales = mk(head_dim // 2), mk(head_dim // 16)

    @classmethod
    def from_planes(cls, k_codes, k_scales, v_codes, v_scales):
        self = cls.__new__(cls)
        self.num_kv_heads, self.capacity, half = v_codes.shape
        self.head_dim = 2 * half
        self.kv_format = "k8v4" if k_scales.dim() == 2 else "nvfp4"
        self.k_codes, self.k_scales, self.v_codes, self.v_scales = k_codes, k_scales, v_codes, v_scales
        return self

    def clone(self):
        return KVPool.from_planes(self.k_codes.clone(), self.k_scales.clone(), self.v_codes.clone(),
                                  self.v_scales.clone())

    @property
    def nbytes(self) -> int:
        return sum(t.numel() * t.element_size() for t in (self.k_codes, self.k_scales, self.v_codes, self.v_scales))

    def desc(self) -> CacheDesc:
        return CacheDesc(self.k_codes.data_ptr(), self.k_scales.data_ptr(), self.v_codes.data_ptr(),
                         self.v_scales.data_ptr(), self.num_kv_heads, self.head_dim, self.capacity,
                         KV_FORMATS[self.kv_format])


def calibrate(pool: KVPool, k_rows: torch.Tensor, v_rows: torch.Tensor, n_rows, out: torch.Tensor | None = None,
              stream=None) -> torch.Tensor:
    """Global scales g[b][h][0|1] = fp32(amax/2688) from bf16 rows [sum n_rows][Hkv][D]."""
    B = len(n_rows)
    if out is None:
        out = torch.empty((B, pool.num_kv_heads, 2), dtype=torch.float32, device=k_rows.device)
    d = pool.desc()
    _check(load_library().nvfp4_kv_calibrate(ctypes.byref(d), _ptr(k_rows), _ptr(v_rows), B, _i64(n_rows),
                                             _ptr(out), _stream(stream)))
    return out


def append(pool: KVPool, k_new: torch.Tensor, v_new: torch.Tensor, global_scale: torch.Tensor, seq_base,
           write_pos, n_new, stream=None) -> None:
    """Quantise n_new[b] bf16 rows per sequence into slots seq_base[b] + write_pos[b] + r."""
    d = pool.desc()
    _check(load_library().nvfp4_kv_append(ctypes.byref(d), _ptr(k_new), _ptr(v_new), _ptr(global_scale),
                                          len(n_new), _i64(seq_base), _i64(write_pos), _i64(n_new),
                                          _stream(stream)))


def workspace_bytes(pool: KVPool, seq_len, n_q: int, num_q_heads: int) -> int:
    d = pool.desc()
    return int(load_library().nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), len(seq_len), _i64(seq_len),
                                                                n_q, num_q_heads))


def alloc_workspace(pool: KVPool, seq_len, n_q: int, num_q_heads: int, device="cuda") -> torch.Tensor:
    nb = workspace_bytes(pool, seq_len, n_q, num_q_heads)
    if nb == 0:
        raise Nvfp4Error(EINVAL, "workspace size query rejected the arguments")
    return torch.empty(nb, dtype=torch.uint8, device=device)


def decode_attn(pool: KVPool, global_scale: torch.Tensor, q: torch.Tensor, seq_base, seq_len, sm_scale: float,
                out: torch.Tensor | None = None, out_dtype=torch.float32, workspace: torch.Tensor | None = None,
                stream=None) -> torch.Tensor:
    """Decode attention; q bf16 [B][n_q][Hq][D] -> out [B][n_q][Hq][D] (fp32 or bf16)."""
    B, n_q, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=out_dtype, device=q.device)
    code = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    if workspace is None:
        workspace = alloc_workspace(pool, seq_len, n_q, Hq, q.device)
    d = pool.desc()
    _check(load_library().nvfp4_decode_attn(ctypes.byref(d), _ptr(global_scale), _ptr(q), _ptr(out), code, B,
                                            _i64(seq_base), _i64(seq_len), n_q, Hq, float(sm_scale),
                                            _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_step(pool: KVPool, global_scale: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                seq_base, seq_len, sm_scale: float, out: torch.Tensor | None = None, out_dtype=torch.float32,
                workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """One decode step: store the n_q new K/V rows per sequence (k_new, v_new bf16 [B*n_q][Hkv][D] at slots
    seq_base + seq_len - n_q + r), then attend; q bf16 [B][n_q][Hq][D] -> out [B][n_q][Hq][D]."""
    B, n_q, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=out_dtype, device=q.device)
    code = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    if workspace is None:
        workspace = alloc_workspace(pool, seq_len, n_q, Hq, q.device)
    d = pool.desc()
    _check(load_library().nvfp4_decode_step(ctypes.byref(d), _ptr(global_scale), _ptr(k_new), _ptr(v_new), _ptr(q),
                                            _ptr(out), code, B, _i64(seq_base), _i64(seq_len), n_q, Hq,
                                            float(sm_scale), _ptr(workspace), workspace.numel(), _stream(stream)))
    return out


def decode_step_noalloc(pool: KVPool, global_scale: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                        q: torch.Tensor, seq_base, seq_len, sm_scale: float, out: torch.Tensor,
                        stream=None) -> torch.Tensor:
    """decode_step without a workspace: the partials go to the library's static per-GPU scratch
    array (nothing is allocated; `out` must be given). Calls that overlap on one GPU race."""
    B, n_q, Hq, D = q.shape
    code = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    d = pool.desc()
    _check(load_library().nvfp4_decode_step_noalloc(ctypes.byref(d), _ptr(global_scale), _ptr(k_new), _ptr(v_new),
                                                    _ptr(q), _ptr(out), code, B, _i64(seq_base), _i64(seq_len), n_q,
                                                    Hq, float(sm_scale), _stream(stream)))
    return out


def decode_step_dev_len(pool: KVPool, global_scale: torch.Tensor, k_new, v_new, q: torch.Tensor, seq_base, max_len,
                        seq_len_dev: torch.Tensor, sm_scale: float, out: torch.Tensor | None = None,
                        out_dtype=torch.float32, workspace: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """decode_step with the lengths in device memory (int64 tensor [B] on the GPU, read when the kernels
    run), so that a captured graph replays across steps; max_len (host) bounds every length and fixes the
    launch. k_new / v_new may both be None (attention only)."""
    B, n_q, Hq, D = q.shape
    if out is None:
        out = torch.empty((B, n_q, Hq, D), dtype=out_dtype, device=q.device)
    code = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    if workspace is None:
        workspace = alloc_workspace(pool, max_len, n_q, Hq, q.device)
    d = pool.desc()
    _check(load_library().nvfp4_decode_step_dev_len(
        ctypes.byref(d), _ptr(global_scale), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out), code, B, _i64(seq_base),
        _i64(max_len), _ptr(seq_len_dev), n_q, Hq, float(sm_scale), _ptr(workspace), workspace.numel(),
        _stream(stream)))
    return out


def decode_attn_partial(pool: KVPool, global_scale, q, seq_base, seq_len, sm_scale: float, workspace,
                        stream=None) -> None:
    B, n_q, Hq, D = q.shape
    d = pool.desc()
    _check(load_library().nvfp4_decode_attn_partial(ctypes.byref(d), _ptr(global_scale), _ptr(q), B,
                                                    _i64(seq_base), _i64(seq_len), n_q, Hq, float(sm_scale),
                                                    _ptr(workspace), workspace.numel(), _stream(stream)))


def decode_attn_combine(pool: KVPool, global_scale, out, seq_len, workspace, stream=None) -> None:
    B, n_q, Hq, D = out.shape
    code = OUT_BF16 if out.dtype == torch.bfloat16 else OUT_F32
    d = pool.desc()
    _check(load_library().nvfp4_decode_attn_combine(ctypes.byref(d), _ptr(global_scale), _ptr(out), code, B,
                                                    _i64(seq_len), n_q, Hq, _ptr(workspace), workspace.numel(),
                                                    _stream(stream)))


def hbm_read_probe(buf: torch.Tensor, workgroups: int, sink: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """Streaming-read probe over the bytes of `buf` (device, 16-byte aligned, size a multiple of 16);
    returns the sink (uint32 [workgroups], a checksum). Timing it gives the plain streaming read rate."""
    if sink is None:
        sink = torch.empty(workgroups, dtype=torch.int32, device=buf.device)
    nbytes = buf.numel() * buf.element_size()
    _check(load_library().nvfp4_hbm_read_probe(_ptr(buf), nbytes, _ptr(sink), int(workgroups), _stream(stream)))
    return sink
