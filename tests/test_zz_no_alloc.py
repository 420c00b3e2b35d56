"""nvfp4_decode_step_noalloc: the decode step with its partials in the library's static
per-GPU scratch array, for callers that cannot allocate. Checked through the C ABI against
nvfp4_decode_step (the entry point it varies) on two calls in a row, the second with a
smaller input: identical pool bytes, the same output (bit for bit where the kernels'
block partition is fixed, to the attention tolerance where waves claim blocks), and both
within the attention tolerance of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from helpers import TOL_REL, OracleRun, assert_planes_equal, assert_same_output, max_err

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qk():
    import quantized_kv_decode_amd as qk
    qk.load_library()
    return qk


def _prepared(qk, w, ref):
    """A pool holding each sequence's first L - n_q rows, and the step's n_q new rows."""
    kd, vd = ref.k.cuda(), ref.v.cuda()
    lens = list(w.seq_lens)
    pool = qk.KVPool(w.num_kv_heads, w.head_dim, w.capacity, device="cuda")
    g = qk.calibrate(pool, kd, vd, lens)
    pre = [L - w.n_q for L in lens]
    rows = lambda t, lo, hi: torch.cat([t[w.seq_base[b] + lo[b]:w.seq_base[b] + hi[b]]
                                        for b in range(w.batch)]).contiguous()
    zero = [0] * w.batch
    qk.append(pool, rows(kd, zero, pre), rows(vd, zero, pre), g, w.seq_base, zero, pre)
    return pool, g, rows(kd, pre, lens), rows(vd, pre, lens)


def _copy(qk, p):
    return qk.KVPool.from_planes(p.k_codes.clone(), p.k_scales.clone(), p.v_codes.clone(), p.v_scales.clone())


def test_noalloc_step_matches_decode_step_twice(qk):
    shapes = [dict(seq_lens=(5000, 1234), num_kv_heads=4, num_q_heads=24, head_dim=256, n_q=6),    # 36 rows
              dict(seq_lens=(700, 129), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=4)]      # smaller
    for shape in shapes:
        w = workloads.small(**shape)
        print("[no-alloc]", shape, flush=True)
        ref = OracleRun(w)
        pool, g, k_step, v_step = _prepared(qk, w, ref)
        pool_a, pool_b = _copy(qk, pool), _copy(qk, pool)
        q = ref.q.cuda()
        lens = list(w.seq_lens)
        out_a = qk.decode_step(pool_a, g, k_step, v_step, q, w.seq_base, lens, w.sm_scale)
        out_b = torch.full_like(out_a, float("nan"))
        qk.decode_step_noalloc(pool_b, g, k_step, v_step, q, w.seq_base, lens, w.sm_scale, out=out_b)
        torch.cuda.synchronize()
        for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
            assert torch.equal(getattr(pool_a, name), getattr(pool_b, name)), name
        assert_same_output(out_a, out_b, w, ref.vmax())
        assert_planes_equal(pool_b, ref.cache)
        exp = ref.attention()
        err, tol = max_err(out_b.cpu().numpy(), exp), TOL_REL * ref.vmax()
        print(f"[no-alloc]   max err {err:.3e}  tol {tol:.3e}", flush=True)
        assert err <= tol


def test_noalloc_rejects_steps_beyond_the_scratch(qk):
    """8192 query rows per KV head over four KV heads need 4 units x 8192 rows x (256 + 2)
    floats of partials, above the 32 MiB array: rejected before any launch."""
    lib = qk.load_library()
    d = qk.CacheDesc(0x100000, 0x110000, 0x120000, 0x130000, 4, 256, 100000)
    rc = lib.nvfp4_decode_step_noalloc(ctypes.byref(d), 0x400000, 0x600000, 0x600000, 0x200000, 0x300000, 0, 1,
                                       qk._i64([0]), qk._i64([20000]), 8192, 4, 0.0625, None)
    assert rc == qk.EWORKSPACE
    assert "scratch" in lib.nvfp4_last_error().decode()
    need = lib.nvfp4_decode_attn_workspace_bytes(ctypes.byref(d), 1, qk._i64([20000]), 8192, 4)
    assert need > 32 << 20
