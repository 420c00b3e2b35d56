"""GPU parity of the K8V4 path (8-bit K, NVFP4 V; knoopx/ninfer page, "Capabilities and
limits", KV storage list) through the C ABI against the fp64 oracle: K rows row-scaled FP8
E4M3 (s = fp32(amax_row / 448), codes nearest E4M3 of |x| / s, ties to even), V NVFP4.

Quantiser: bit-exact planes (K codes and fp32 row scales, V codes and scales). Attention:
max |o_gpu - o_ref| <= 2e-3 * max |V_hat| over the test case, on the shapes of every decode
kernel variant (one to four row tiles, head_dim 128 and 256, row chunks of wide draft windows
and prefill), the fused decode step, the device-length step and the five configurations at
full size through the timed step.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import TOL_REL, OracleRun, assert_planes_equal, assert_same_output, gpu_run
from test_gpu_parity import (DEV_LEN_CASES, _assert_seq_slots_equal, _check_decode, _full_step, _seq_rows,
                             _spaced_pool, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qk():
    import quantized_kv_decode_amd as qk
    qk.load_library()
    return qk


def k8(shape):
    return workloads.small(**shape, kv_format="k8v4")


APPEND_SHAPES = [
    dict(seq_lens=(200, 77), num_kv_heads=2, num_q_heads=6, head_dim=256, n_q=3),
    dict(seq_lens=(45,), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=1, v_dist="laplace"),
    dict(seq_lens=(300, 1, 64, 33), num_kv_heads=4, num_q_heads=8, head_dim=256, n_q=1, outlier_frac=0.02),
]


@pytest.mark.parametrize("shape", APPEND_SHAPES)
def test_k8v4_calibrate_and_append_bit_exact(qk, shape):
    w = k8(shape)
    say("k8v4 calibrate/append", shape)
    ref = OracleRun(w)
    pool, g, _ = gpu_run(w, ref.k, ref.v, ref.q)
    assert np.array_equal(g.cpu().numpy(), ref.g)
    assert_planes_equal(pool, ref.cache)


def _fp8_adversarial_rows(D):
    """K rows whose scale is a power of two (amax 448 * 2^k) and whose elements sit on every
    E4M3 midpoint and one bf16 step either side, plus zero, -0, subnormal-maximum and
    largest-bf16 rows, and rows of random magnitude over 60 decades."""
    e4 = [oracle.e4m3_value(c) for c in range(127)]
    rows = []
    for k in (-20, -6, 0, 5, 17):
        mids = np.array([(e4[i] + e4[i + 1]) / 2 * 2.0 ** k for i in range(126)], np.float32)
        mb = (np.frombuffer(mids.tobytes(), np.uint32) >> 16).astype(np.uint16)
        vals = np.concatenate([mb, mb + 1, mb - 1]).astype(np.uint16)
        top = (np.frombuffer(np.array([448 * 2.0 ** k], np.float32).tobytes(), np.uint32) >> 16)[0]
        for i in range(0, vals.size, D - 1):
            row = np.zeros(D, np.uint16)
            row[0] = top
            chunk = vals[i:i + D - 1]
            row[1:1 + chunk.size] = chunk | (np.arange(chunk.size, dtype=np.uint16) % 2 << 15)
            rows.append(row)
    edge = np.zeros((4, D), np.uint16)
    edge[1, :] = 0x8000
    edge[2, 5] = 0x0001
    edge[3, 7] = 0x7F7F
    rows += list(edge)
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((64, D)) * 10.0 ** rng.uniform(-30, 30, (64, 1))).astype(np.float32)
    rows += list((np.frombuffer(x.tobytes(), np.uint32) >> 16).astype(np.uint16).reshape(64, D))
    return np.stack(rows)


@pytest.mark.parametrize("D", [128, 256])
def test_k8v4_append_adversarial_rows(qk, D):
    rows = _fp8_adversarial_rows(D)
    n = rows.shape[0]
    say("k8v4 adversarial append", D, n, "rows")
    x = workloads.from_u16(rows).reshape(n, 1, D)
    g = np.array([[[0.37, 0.002]]], np.float32)
    ref = oracle.Cache(1, D, n, kv_format="k8v4")
    oracle.append(ref, workloads.as_u16(x), workloads.as_u16(x), g, [0], [0], [n])
    pool = qk.KVPool(1, D, n, kv_format="k8v4")
    xd = x.cuda()
    qk.append(pool, xd, xd, torch.from_numpy(g).cuda(), [0], [0], [n])
    torch.cuda.synchronize()
    assert_planes_equal(pool, ref)


def test_k8v4_append_in_chunks_at_offsets(qk):
    w = k8(dict(seq_lens=(130, 70), num_kv_heads=2, num_q_heads=4, head_dim=256, n_q=2))
    say("k8v4 chunked append")
    ref = OracleRun(w)
    pool, _, _ = gpu_run(w, ref.k, ref.v, ref.q, chunk_rows=17)
    assert_planes_equal(pool, ref.cache)


DECODE_SHAPES = [
    dict(seq_lens=(512,), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=1),                     # 4 rows, D 128
    dict(seq_lens=(1000, 77, 3), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=1),             # 6 rows
    dict(seq_lens=(700, 129), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=4, v_dist="laplace"),  # 24 rows
    dict(seq_lens=(1500, 45), num_kv_heads=2, num_q_heads=8, head_dim=128, n_q=5),                 # 20 rows, D 128
    dict(seq_lens=(963,), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=6, outlier_frac=0.02),  # 36 rows
    dict(seq_lens=(6, 7, 31, 32, 33), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=6),
    dict(seq_lens=(257,), num_kv_heads=1, num_q_heads=8, head_dim=128, n_q=6),                     # 48 rows, D 128
    dict(seq_lens=(333, 100), num_kv_heads=1, num_q_heads=16, head_dim=256, n_q=4),                # 64 rows
    dict(seq_lens=(1234,), num_kv_heads=2, num_q_heads=16, head_dim=256, n_q=4, outlier_frac=0.02),  # 32 rows
    dict(seq_lens=(700, 129), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=16),               # 96: 3 chunks
    dict(seq_lens=(900, 40), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=12, v_dist="laplace"),  # 72
    dict(seq_lens=(600,), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=64),                    # 384: prefill
    dict(seq_lens=(300, 1000), num_kv_heads=2, num_q_heads=8, head_dim=128, n_q=100),              # 400, ragged
]


@pytest.mark.parametrize("shape", DECODE_SHAPES)
def test_k8v4_decode_matches_oracle(qk, shape):
    w = k8(shape)
    say("k8v4 decode", shape)
    ref = OracleRun(w)
    pool, g, out = gpu_run(w, ref.k, ref.v, ref.q)
    assert_planes_equal(pool, ref.cache)
    _check_decode(w, ref, out)


@pytest.mark.parametrize("shape", [DECODE_SHAPES[i] for i in (1, 2, 4, 7, 9)] + [
    dict(seq_lens=(4003, 161, 4), num_kv_heads=4, num_q_heads=24, head_dim=256, n_q=4)])
def test_k8v4_decode_step_equals_append_then_decode(qk, shape):
    w = k8(shape)
    say("k8v4 decode step", shape)
    ref = OracleRun(w)
    kd, vd = ref.k.cuda(), ref.v.cuda()
    lens = list(w.seq_lens)
    pool = qk.KVPool(w.num_kv_heads, w.head_dim, w.capacity, device="cuda", kv_format="k8v4")
    g = qk.calibrate(pool, kd, vd, lens)
    pre = [L - w.n_q for L in lens]
    zero = [0] * w.batch
    qk.append(pool, _seq_rows(kd, w, zero, pre), _seq_rows(vd, w, zero, pre), g, w.seq_base, zero, pre)
    k_step, v_step = _seq_rows(kd, w, pre, lens), _seq_rows(vd, w, pre, lens)
    pool_a, pool_b = pool.clone(), pool.clone()
    q = ref.q.cuda()
    qk.append(pool_a, k_step, v_step, g, w.seq_base, pre, [w.n_q] * w.batch)
    out_a = qk.decode_attn(pool_a, g, q, w.seq_base, lens, w.sm_scale)
    out_b = qk.decode_step(pool_b, g, k_step, v_step, q, w.seq_base, lens, w.sm_scale)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        assert torch.equal(getattr(pool_a, name), getattr(pool_b, name)), name
    assert_same_output(out_a, out_b, w, ref.vmax())
    assert_planes_equal(pool_b, ref.cache)
    _check_decode(w, ref, out_b)


@pytest.mark.parametrize("shape,extra", [DEV_LEN_CASES[i] for i in (1, 2, 3, 4, 7, 10, 11, 13)])
def test_k8v4_decode_step_device_lengths(qk, shape, extra):
    w = k8(shape)
    say("k8v4 decode step, device lengths", shape, "bound +", extra)
    ref = OracleRun(w)
    max_len = [L + extra for L in w.seq_lens]
    pool, base = _spaced_pool(qk, w, max_len)
    kd, vd = ref.k.cuda(), ref.v.cuda()
    g = qk.calibrate(pool, kd, vd, list(w.seq_lens))
    lens = list(w.seq_lens)
    pre = [L - w.n_q for L in lens]
    zero = [0] * w.batch
    qk.append(pool, _seq_rows(kd, w, zero, pre), _seq_rows(vd, w, zero, pre), g, base, zero, pre)
    lens_dev = torch.tensor(lens, dtype=torch.int64, device="cuda")
    out = qk.decode_step_dev_len(pool, g, _seq_rows(kd, w, pre, lens), _seq_rows(vd, w, pre, lens), ref.q.cuda(),
                                 base, max_len, lens_dev, w.sm_scale)
    torch.cuda.synchronize()
    _assert_seq_slots_equal(pool, base, ref, w)
    _check_decode(w, ref, out)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", workloads.ORDER_K8V4)
def test_k8v4_full_workload_step(qk, name):
    """The five configurations stored as K8V4, at full size through the timed decode step:
    planes bit-exact, every query row within tolerance."""
    w = workloads.get(name)
    say("full workload", name, w.seq_lens, "n_q", w.n_q)
    ref = OracleRun(w)
    pool, g, out, out_dl = _full_step(qk, w, ref)
    assert_planes_equal(pool, ref.cache)
    _check_decode(w, ref, out)
    if out_dl is not None:
        _check_decode(w, ref, out_dl)
