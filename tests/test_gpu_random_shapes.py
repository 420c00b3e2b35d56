"""A seeded sweep of random decode shapes through the fused decode step (the call the
benchmark times), NVFP4 and K8V4 pools: one to four row tiles, row chunks above 64 rows,
head_dim 128 and 256, ragged batches of one to eight sequences, outlier channels and
Laplace V. Every case: pool planes bit-exact against the fp64 oracle's, every query row
within the attention tolerance.
"""
import numpy as np
import pytest
import torch

import workloads
from helpers import OracleRun, assert_planes_equal
from test_gpu_parity import _check_decode, _seq_rows, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qk():
    import quantized_kv_decode_amd as qk
    qk.load_library()
    return qk


def _shapes(n=60, seed=2026):
    """n shapes, the row classes (1-16, 17-32, 33-48, 49-64 and 65-128 query rows per KV
    head: one to four row tiles, then row chunks) in turn."""
    rng = np.random.default_rng(seed)
    classes = [(1, 16), (17, 32), (33, 48), (49, 64), (65, 128)]
    out = []
    for i in range(n):
        lo, hi = classes[i % len(classes)]
        while True:
            G = int(rng.choice([1, 2, 3, 4, 6, 8]))
            cands = [q for q in range(1, 65) if lo <= G * q <= hi]
            if cands:
                n_q = int(rng.choice(cands))
                break
        D = int(rng.choice([128, 256]))
        Hkv = int(rng.choice([1, 2, 4]))
        B = int(rng.integers(1, 9))
        lens = tuple(int(v) for v in rng.integers(n_q, 1500, B))
        out.append(dict(seq_lens=lens, num_kv_heads=Hkv, num_q_heads=Hkv * G, head_dim=D, n_q=n_q,
                        v_dist=str(rng.choice(["normal", "laplace"])),
                        outlier_frac=float(rng.choice([0.0, 0.0, 0.02])),
                        kv_format=str(rng.choice(["nvfp4", "k8v4"]))))
    return out


@pytest.mark.parametrize("shape", _shapes(), ids=lambda s: f"{s['kv_format']}-D{s['head_dim']}-B{len(s['seq_lens'])}-"
                                                          f"R{s['num_q_heads'] // s['num_kv_heads'] * s['n_q']}")
def test_random_shape_decode_step(qk, shape):
    w = workloads.small(**shape)
    say("random shape", shape)
    ref = OracleRun(w)
    kd, vd = ref.k.cuda(), ref.v.cuda()
    lens = list(w.seq_lens)
    pool = qk.KVPool(w.num_kv_heads, w.head_dim, w.capacity, device="cuda", kv_format=w.kv_format)
    g = qk.calibrate(pool, kd, vd, lens)
    pre = [L - w.n_q for L in lens]
    zero = [0] * w.batch
    qk.append(pool, _seq_rows(kd, w, zero, pre), _seq_rows(vd, w, zero, pre), g, w.seq_base, zero, pre)
    out = qk.decode_step(pool, g, _seq_rows(kd, w, pre, lens), _seq_rows(vd, w, pre, lens), ref.q.cuda(),
                         w.seq_base, lens, w.sm_scale)
    torch.cuda.synchronize()
    assert np.array_equal(g.cpu().numpy(), ref.g)
    assert_planes_equal(pool, ref.cache)
    _check_decode(w, ref, out)
