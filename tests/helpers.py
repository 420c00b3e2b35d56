"""Shared test plumbing: run a workload through the oracle and through the HIP path.

The oracle side and the GPU side only share the seeded inputs from `workloads`.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle
import workloads

# Attention acceptance: max |o_gpu - o_ref| <= TOL_REL * max |V_hat| over the test case.
TOL_REL = 2e-3


class OracleRun:
    def __init__(self, w: workloads.Workload, k=None, v=None, q=None, nthreads=None):
        self.w = w
        self.k = workloads.all_kv_rows(w, "k") if k is None else k          # bf16 [cap][Hkv][D]
        self.v = workloads.all_kv_rows(w, "v") if v is None else v
        self.q = workloads.queries(w) if q is None else q
        ku, vu = workloads.as_u16(self.k), workloads.as_u16(self.v)
        self.g = oracle.calibrate(ku, vu, w.seq_lens)
        self.cache = oracle.Cache(w.num_kv_heads, w.head_dim, w.capacity, kv_format=w.kv_format)
        oracle.append(self.cache, ku, vu, self.g, w.seq_base, [0] * w.batch, list(w.seq_lens), nthreads)
        self.nthreads = nthreads

    def attention(self, sel=None):
        return oracle.attention(self.cache, self.g, workloads.as_u16(self.q), self.w.seq_base, self.w.seq_lens,
                                self.w.n_q, self.w.sm_scale, sel=sel, nthreads=self.nthreads)

    def vmax(self) -> float:
        """max |V_hat| over every stored V row of the test case."""
        m = 0.0
        w = self.w
        for b in range(w.batch):
            for h in range(w.num_kv_heads):
                base, L = w.seq_base[b], w.seq_lens[b]
                gv = float(self.g[b, h, 1])
                codes = self.cache.v_codes[h, base:base + L]
                scales = self.cache.v_scales[h, base:base + L].astype(np.int64)
                # max |e2m1| per byte is max of the two nibbles' magnitudes; E4M3 scale value
                mag = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
                lo = mag[codes & 7]
                hi = mag[(codes >> 4) & 7]
                emax = np.maximum(lo, hi).reshape(L, -1, 8).max(axis=2)       # per group
                sval = np.array([oracle.e4m3_value(c) for c in range(256)])[scales]
                m = max(m, float((emax * sval).max() * gv))
        return m


def gpu_run(w: workloads.Workload, k: torch.Tensor, v: torch.Tensor, q: torch.Tensor, out_dtype=torch.float32,
            chunk_rows: int | None = None):
    """Calibrate, append and decode on the GPU through the C ABI. Returns (pool, g, out)."""
    import quantized_kv_decode_amd as qk
    dev = "cuda"
    pool = qk.KVPool(w.num_kv_heads, w.head_dim, w.capacity, device=dev, kv_format=w.kv_format)
    kd, vd = k.to(dev), v.to(dev)
    g = qk.calibrate(pool, kd, vd, list(w.seq_lens))
    if chunk_rows is None:
        qk.append(pool, kd, vd, g, w.seq_base, [0] * w.batch, list(w.seq_lens))
    else:
        for b in range(w.batch):
            base, L = w.seq_base[b], w.seq_lens[b]
            for r0 in range(0, L, chunk_rows):
                r1 = min(L, r0 + chunk_rows)
                ks = kd[base + r0:base + r1].contiguous()
                vs = vd[base + r0:base + r1].contiguous()
                n_new = [0] * w.batch
                n_new[b] = r1 - r0
                wp = [0] * w.batch
                wp[b] = r0
                qk.append(pool, ks, vs, g, w.seq_base, wp, n_new)
    del kd, vd
    out = qk.decode_attn(pool, g, q.to(dev), w.seq_base, list(w.seq_lens), w.sm_scale, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return pool, g, out


def assert_planes_equal(pool, cache: oracle.Cache):
    """Every plane byte for byte (K8V4's fp32 row scales compared as bit patterns)."""
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        got = getattr(pool, name).cpu().numpy()
        ref = getattr(cache, name)
        if got.dtype == np.float32:
            got, ref = got.view(np.uint32), ref.view(np.uint32)
        if not np.array_equal(got, ref):
            bad = np.argwhere(got != ref)
            i = tuple(bad[0])
            raise AssertionError(f"{name}: {len(bad)} values differ; first at {i}: gpu {got[i]:#x} oracle {ref[i]:#x}")


def max_err(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.abs(got.astype(np.float64) - ref).max())


def _bf16_u16(x):
    return workloads.as_u16(torch.tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16))


def _bf16_neighbours(vals):
    """Every bf16 value in vals plus the bf16 values one ulp either side."""
    u = _bf16_u16(vals).astype(np.int32)
    out = np.concatenate([u, u + 1, np.maximum(u - 1, 0)]) & 0x7FFF
    sign = np.arange(out.size) % 2 == 1
    return (out | (sign.astype(np.int32) << 15)).astype(np.uint16)


def adversarial_rows(D=256):
    """Groups whose maxima sit on every E4M3 midpoint (times 6) and whose elements sit
    on every E2M1 midpoint of their scale, with bf16 neighbours, signed zeros, zero
    groups and saturating values, for g = 1 (so every tie is representable)."""
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    groups = []
    for k in range(126):                                     # scale ties and their neighbours
        mid = 0.5 * (e4[k] + e4[k + 1])
        amax = _bf16_neighbours([6 * mid])
        for a in amax:
            grp = np.zeros(16, np.uint16)
            grp[0] = a
            grp[1] = _bf16_u16([-mid])[0]
            groups.append(grp)
    thr = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.5, 1.0, 3.0, 6.0]
    for c in (1, 2, 7, 8, 0x30, 0x38, 0x3A, 0x55, 0x70, 0x7E):   # element ties under several scales
        S = e4[c]
        vals = _bf16_neighbours([t * S for t in thr])
        for i in range(0, vals.size, 15):
            grp = np.zeros(16, np.uint16)
            grp[0] = _bf16_u16([6 * S])[0]
            chunk = vals[i:i + 15]
            grp[1:1 + chunk.size] = chunk
            groups.append(grp)
    groups.append(np.zeros(16, np.uint16))                     # +0 group
    groups.append(np.full(16, 0x8000, np.uint16))              # -0 group
    groups.append(_bf16_u16([3e4, -3e4, 1e5, 7, -1e-3] + [0] * 11))    # saturating
    groups.append(_bf16_u16([1e-38, -3e-39, 1e-40] + [0] * 13))        # bf16 subnormals
    n = len(groups)
    per_row = D // 16
    rows = int(math.ceil(n / per_row))
    flat = np.zeros((rows * per_row, 16), np.uint16)
    flat[:n] = np.stack(groups)
    return flat.reshape(rows, D)


def deterministic(w) -> bool:
    """Whether the decode kernels give the same output bits on every run for this shape: one
    row tile (up to 16 query rows per KV head) processes a fixed block partition; at two row
    tiles (17-32 rows, and the 32-row chunks above 64 rows) the waves, and in the wave-pair
    kernel (33-64 rows) the pairs, claim blocks as they free up, so the partition -- and the
    fp16 rounding of the probabilities against each wave's or pair's reference -- depends on
    timing."""
    return w.rows <= 16


def assert_same_output(a: torch.Tensor, b: torch.Tensor, w, vmax: float):
    """Outputs of two runs of the same step: identical bits where the kernels are
    deterministic, else within the attention tolerance of each other."""
    if deterministic(w):
        assert torch.equal(a, b)
    else:
        err = (a.float() - b.float()).abs().max().item()
        assert err <= TOL_REL * vmax, (err, TOL_REL * vmax)
