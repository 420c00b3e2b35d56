"""GPU parity: the HIP path through the C ABI against the fp64 CPU oracle.

Quantiser (calibrate + append): bit-exact bytes. Attention: max |o_gpu - o_ref|
<= 2e-3 * max |V_hat| over the test case (fp32 accumulation against fp64 over
the same dequantised KV, which the oracle builds from its own quantiser).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from helpers import (TOL_REL, OracleRun, _bf16_u16, adversarial_rows, assert_planes_equal, assert_same_output,
                     deterministic, gpu_run, max_err)

pytestmark = pytest.mark.gpu


def say(*a):
    print("[gpu-parity]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def qk():
    import quantized_kv_decode_amd as qk
    qk.load_library()
    return qk


# ---------------------------------------------------------------- quantiser ------
SMALL = [
    dict(seq_lens=(200, 77), num_kv_heads=2, num_q_heads=6, head_dim=256, n_q=3),
    dict(seq_lens=(45,), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=1, v_dist="laplace"),
    dict(seq_lens=(300, 1, 64, 33), num_kv_heads=4, num_q_heads=8, head_dim=256, n_q=1, outlier_frac=0.02),
]


@pytest.mark.parametrize("shape", SMALL)
def test_calibrate_and_append_bit_exact(qk, shape):
    w = workloads.small(**shape)
    say("calibrate/append", shape)
    ref = OracleRun(w)
    pool, g, _ = gpu_run(w, ref.k, ref.v, ref.q)
    assert np.array_equal(g.cpu().numpy(), ref.g), "global scales differ"
    assert_planes_equal(pool, ref.cache)


def test_append_in_chunks_at_offsets(qk):
    w = workloads.small(seq_lens=(130, 70), num_kv_heads=2, num_q_heads=4, head_dim=256, n_q=2)
    say("chunked append")
    ref = OracleRun(w)
    pool, _, _ = gpu_run(w, ref.k, ref.v, ref.q, chunk_rows=17)
    assert_planes_equal(pool, ref.cache)


@pytest.mark.parametrize("gval", [1.0, 0.5, 3.0, 0.0, 1e-30, 7.1e-36, 1e-40, 2.5e30])
def test_append_adversarial_groups(qk, gval):
    D = 256
    rows = adversarial_rows(D)
    n = rows.shape[0]
    say("adversarial append", gval, n, "rows")
    # the same rows for K and V, one KV head, one sequence
    x = workloads.from_u16(rows).reshape(n, 1, D)
    g = np.array([[[gval, gval]]], np.float32)
    ref = oracle.Cache(1, D, n)
    oracle.append(ref, workloads.as_u16(x), workloads.as_u16(x), g, [0], [0], [n])
    pool = qk.KVPool(1, D, n)
    xd = x.cuda()
    qk.append(pool, xd, xd, torch.from_numpy(g).cuda(), [0], [0], [n])
    torch.cuda.synchronize()
    assert_planes_equal(pool, ref)


@pytest.mark.parametrize("kv_format", ["nvfp4", "k8v4"])
def test_append_mixed_scale_ranges_in_one_wave(qk, kv_format):
    """Ragged sequences whose global scales alternate between the fast path's range and
    outside it (1e-40, 2.5e30, 0: the exact decision), so that lanes of one wave (four rows of
    one plane at head_dim 256) take different paths; planes bit-exact against the oracle."""
    D, H = 256, 2
    lens = [3, 5, 2, 6, 1, 7]
    n = sum(lens)
    rows = adversarial_rows(D)
    reps = -(-n * H // rows.shape[0])
    x = workloads.from_u16(np.tile(rows, (reps, 1))[:n * H]).reshape(n, H, D)
    gvals = [1.0, 1e-40, 2.5e30, 0.37, 0.0, 3.0, 7.1e-36, 0.002]
    g = np.array([[[gvals[(2 * b + h + kv) % len(gvals)] for kv in range(2)] for h in range(H)]
                  for b in range(len(lens))], np.float32)
    say("mixed-range append", kv_format, lens)
    base = [0] + [int(v) for v in np.cumsum(lens)[:-1]]
    ref = oracle.Cache(H, D, n, kv_format=kv_format)
    xu = workloads.as_u16(x)
    oracle.append(ref, xu, xu, g, base, [0] * len(lens), lens)
    pool = qk.KVPool(H, D, n, kv_format=kv_format)
    xd = x.cuda()
    qk.append(pool, xd, xd, torch.from_numpy(g).cuda(), base, [0] * len(lens), lens)
    torch.cuda.synchronize()
    assert_planes_equal(pool, ref)


@pytest.mark.parametrize("kv_format", ["nvfp4", "k8v4"])
def test_append_graph_replay(qk, kv_format):
    """The append kernel captured once in a HIP graph and replayed three times, with new rows
    and new global scales copied into the same buffers between replays (eager work and a
    synchronisation between them): after every replay the pool holds the oracle's bytes for
    that replay's rows at slots [10, 50), and zeros elsewhere."""
    D, H, n, cap = 256, 2, 40, 96
    say("append graph replay", kv_format)
    pool = qk.KVPool(H, D, cap, kv_format=kv_format)
    k_buf = torch.zeros((n, H, D), dtype=torch.bfloat16, device="cuda")
    v_buf = torch.zeros_like(k_buf)
    g_buf = torch.zeros((1, H, 2), dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            qk.append(pool, k_buf, v_buf, g_buf, [10], [0], [n])
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(31)
    for rep in range(3):
        k = (torch.randn((n, H, D), generator=gen) * (1 + 3 * rep)).to(torch.bfloat16)
        v = (torch.randn((n, H, D), generator=gen) * 0.1 ** rep).to(torch.bfloat16)
        ku, vu = workloads.as_u16(k), workloads.as_u16(v)
        g = oracle.calibrate(ku, vu, [n])
        k_buf.copy_(k)
        v_buf.copy_(v)
        g_buf.copy_(torch.from_numpy(g))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        ref = oracle.Cache(H, D, cap, kv_format=kv_format)
        oracle.append(ref, ku, vu, g, [10], [0], [n])
        assert_planes_equal(pool, ref)


def test_calibrate_edge_values(qk):
    D = 128
    say("calibrate edges")
    rows = np.zeros((3, 2, D), np.uint16)        # seq 0: 1 row all zero; seq 1: 2 rows
    rows[1, 0, 5] = _bf16_u16([-2688.0])[0]
    rows[2, 1, 7] = _bf16_u16([1e-38])[0]
    rows[2, 0, 9] = _bf16_u16([3.3e38])[0]
    x = workloads.from_u16(rows)
    ref = oracle.calibrate(rows, rows, [1, 2])
    pool = qk.KVPool(2, D, 8)
    g = qk.calibrate(pool, x.cuda(), x.cuda(), [1, 2])
    assert np.array_equal(g.cpu().numpy(), ref)
    # a sequence with no rows gets g = 0
    g0 = qk.calibrate(pool, x.cuda(), x.cuda(), [0, 3])
    assert np.array_equal(g0.cpu().numpy(), oracle.calibrate(rows, rows, [0, 3]))


# ---------------------------------------------------------------- attention ------
DECODE_SHAPES = [
    dict(seq_lens=(512,), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=1),
    dict(seq_lens=(1000, 77, 3), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=1),
    dict(seq_lens=(700, 129), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=4, v_dist="laplace"),   # 24 rows
    dict(seq_lens=(963,), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=6, outlier_frac=0.02),        # 36 rows
    dict(seq_lens=(6, 7, 31, 32, 33), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=6),
    dict(seq_lens=(2050,), num_kv_heads=2, num_q_heads=2, head_dim=128, n_q=5),                            # G = 1
    dict(seq_lens=(333, 100), num_kv_heads=1, num_q_heads=16, head_dim=256, n_q=4),                       # 64 rows
    dict(seq_lens=(257,), num_kv_heads=1, num_q_heads=8, head_dim=128, n_q=6),                            # 48 rows
    dict(seq_lens=(1500, 45), num_kv_heads=2, num_q_heads=8, head_dim=128, n_q=5),                        # 20 rows, D 128
    dict(seq_lens=(1234,), num_kv_heads=2, num_q_heads=16, head_dim=256, n_q=4, outlier_frac=0.02),      # 32 rows
    # wide draft windows: 32-row chunks side by side over one split plan
    dict(seq_lens=(700, 129), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=16),   # 96 rows: 3 chunks
    dict(seq_lens=(900, 40), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=12, v_dist="laplace"),  # 72: 32 + 32 + 8
    dict(seq_lens=(600,), num_kv_heads=1, num_q_heads=16, head_dim=128, n_q=8),         # 128 rows: 4 chunks
    dict(seq_lens=(17, 90), num_kv_heads=1, num_q_heads=5, head_dim=256, n_q=15),      # 75 rows, lengths < 2 blocks
    # prefill chunks: many 32-row chunks side by side, each skipping keys its rows cannot see
    dict(seq_lens=(600,), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=64),        # 384 rows: 12 chunks
    dict(seq_lens=(300, 1000), num_kv_heads=2, num_q_heads=8, head_dim=128, n_q=100),  # 400 rows, ragged
    dict(seq_lens=(2100,), num_kv_heads=4, num_q_heads=24, head_dim=256, n_q=256, v_dist="laplace"),  # 1536 rows
]


def _check_decode(w, ref, out, sel=None):
    got = out.float().cpu().numpy()
    if sel is None:
        exp = ref.attention()
    else:
        exp = ref.attention(sel)
        got = np.stack([got[b, i, h] for (b, i, h) in sel])
    tol = TOL_REL * ref.vmax()
    err = max_err(got, exp)
    say(f"  max err {err:.3e}  tol {tol:.3e}  ({err / tol * 100:.2f}% of budget)")
    assert err <= tol
    return err


@pytest.mark.parametrize("shape", DECODE_SHAPES)
def test_decode_matches_oracle(qk, shape):
    w = workloads.small(**shape)
    say("decode", shape)
    ref = OracleRun(w)
    pool, g, out = gpu_run(w, ref.k, ref.v, ref.q)
    assert_planes_equal(pool, ref.cache)
    _check_decode(w, ref, out)
    # bf16 output is the round-to-nearest-even of the fp32 result (of the same partition: bit
    # for bit where the kernels are deterministic, else one bf16 step at most)
    outb = qk.decode_attn(pool, g, ref.q.cuda(), w.seq_base, list(w.seq_lens), w.sm_scale, out_dtype=torch.bfloat16)
    if deterministic(w):
        assert torch.equal(outb, out.to(torch.bfloat16))
    else:
        o32 = out.float()
        assert ((outb.float() - o32).abs() <= o32.abs() * 2.0 ** -8 + TOL_REL * ref.vmax()).all()


STEP_SHAPES = DECODE_SHAPES + [
    dict(seq_lens=(4003,), num_kv_heads=4, num_q_heads=24, head_dim=256, n_q=6),      # 3-token remainder joins
    dict(seq_lens=(4003, 161, 4), num_kv_heads=4, num_q_heads=24, head_dim=256, n_q=4),
]


@pytest.mark.parametrize("shape", STEP_SHAPES)
def test_decode_step_equals_append_then_decode(qk, shape):
    """The fused step, where the decode kernel stores the step's n_q rows itself, leaves
    the same pool bytes and writes the same output bits as nvfp4_kv_append followed by
    nvfp4_decode_attn, and both match the oracle."""
    w = workloads.small(**shape)
    say("decode step", shape)
    ref = OracleRun(w)
    kd, vd = ref.k.cuda(), ref.v.cuda()
    pool = qk.KVPool(w.num_kv_heads, w.head_dim, w.capacity, device="cuda", kv_format=w.kv_format)
    g = qk.calibrate(pool, kd, vd, list(w.seq_lens))
    pre = [L - w.n_q for L in w.seq_lens]
    sl = lambda t, lo, hi: torch.cat([t[w.seq_base[b] + lo[b]:w.seq_base[b] + hi[b]] for b in range(w.batch)])
    qk.append(pool, sl(kd, [0] * w.batch, pre).contiguous(), sl(vd, [0] * w.batch, pre).contiguous(), g,
              w.seq_base, [0] * w.batch, pre)
    k_step = sl(kd, pre, list(w.seq_lens)).contiguous()
    v_step = sl(vd, pre, list(w.seq_lens)).contiguous()
    copy = lambda p: qk.KVPool.from_planes(p.k_codes.clone(), p.k_scales.clone(), p.v_codes.clone(),
                                           p.v_scales.clone())
    pool_a, pool_b = copy(pool), copy(pool)
    q = ref.q.cuda()
    qk.append(pool_a, k_step, v_step, g, w.seq_base, pre, [w.n_q] * w.batch)
    out_a = qk.decode_attn(pool_a, g, q, w.seq_base, list(w.seq_lens), w.sm_scale)
    out_b = qk.decode_step(pool_b, g, k_step, v_step, q, w.seq_base, list(w.seq_lens), w.sm_scale)
    torch.cuda.synchronize()
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        assert torch.equal(getattr(pool_a, name), getattr(pool_b, name)), name
    assert_same_output(out_a, out_b, w, ref.vmax())
    assert_planes_equal(pool_b, ref.cache)
    _check_decode(w, ref, out_b)


def _spaced_pool(qk, w, max_len):
    """A pool in which sequence b owns slots [base[b], base[b] + max_len[b]): room to grow."""
    base = [int(x) for x in np.concatenate([[0], np.cumsum(max_len)[:-1]])]
    return qk.KVPool(w.num_kv_heads, w.head_dim, int(sum(max_len)), device="cuda", kv_format=w.kv_format), base


def _seq_rows(t, w, lo, hi):
    """Rows [lo[b], hi[b]) of every sequence b of w's row tensor, concatenated over b."""
    return torch.cat([t[w.seq_base[b] + lo[b]:w.seq_base[b] + hi[b]] for b in range(w.batch)]).contiguous()


def _assert_seq_slots_equal(pool, base, ref, w):
    for name in ("k_codes", "k_scales", "v_codes", "v_scales"):
        got = getattr(pool, name).cpu().numpy()
        exp = getattr(ref.cache, name)
        for b in range(w.batch):
            L = w.seq_lens[b]
            assert np.array_equal(got[:, base[b]:base[b] + L], exp[:, w.seq_base[b]:w.seq_base[b] + L]), (name, b)


DEV_LEN_CASES = [
    (dict(seq_lens=(512,), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=1), 0),          # bound = length
    (dict(seq_lens=(1000, 77, 3), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=1), 700),
    (dict(seq_lens=(700, 129), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=4), 3000),   # 24 rows
    (dict(seq_lens=(1500, 45), num_kv_heads=2, num_q_heads=8, head_dim=128, n_q=5), 2500),    # 20 rows, D 128
    (dict(seq_lens=(963,), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=6, outlier_frac=0.02), 5000),
    (dict(seq_lens=(6, 40), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=6), 100000),     # nearly all units empty
    (dict(seq_lens=(9, 20), num_kv_heads=1, num_q_heads=4, head_dim=256, n_q=1), 60000),      # one row tile, same
    (dict(seq_lens=(700, 129), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=16), 2000),  # 96 rows, three chunks
    # 128 rows in 4 chunks: bounds of 500 / 415 tokens plan 3 units per sequence, most of them
    # empty at these lengths, and the combine takes its path for at most one unit per wave
    (dict(seq_lens=(130, 45), num_kv_heads=1, num_q_heads=16, head_dim=128, n_q=8), 370),
    # many query tokens against a bound far above the length: the device splits a short
    # length over many planned units, and every unit must still hold at least n_q tokens so
    # that the step's new rows all fall in the last one (one-wave kernel at 32 rows, the pair
    # kernel at 48 and 64, row chunks at 96 and 128)
    (dict(seq_lens=(200, 77), num_kv_heads=1, num_q_heads=1, head_dim=256, n_q=32), 60000),
    (dict(seq_lens=(300, 97), num_kv_heads=1, num_q_heads=1, head_dim=256, n_q=48), 100000),
    (dict(seq_lens=(300,), num_kv_heads=2, num_q_heads=2, head_dim=128, n_q=64), 100000),
    (dict(seq_lens=(250, 140), num_kv_heads=1, num_q_heads=2, head_dim=256, n_q=48), 50000),
    (dict(seq_lens=(400,), num_kv_heads=1, num_q_heads=1, head_dim=128, n_q=128), 80000),
]


@pytest.mark.parametrize("shape,extra", DEV_LEN_CASES)
def test_decode_step_device_lengths(qk, shape, extra):
    """nvfp4_decode_step_dev_len with lengths in device memory and an upper bound max_len:
    the step's rows land in the same bytes as the oracle's, the output passes the oracle."""
    w = workloads.small(**shape)
    say("decode step, device lengths", shape, "bound +", extra)
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


@pytest.mark.parametrize("n_q", [1, 4, 16])
def test_decode_step_device_lengths_graph_replay(qk, n_q):
    """One HIP graph of the device-length step, captured once and replayed over four decode
    steps while the sequences grow by n_q tokens per step (new q, k_new, v_new and lengths
    written into the same buffers between replays): every replay passes the oracle at its
    lengths, the pool matches the oracle's bytes at the end, and replaying the last step
    again gives identical output bits. n_q = 16 is 96 rows per KV head: three 32-row chunks
    side by side, each storing the step's rows itself."""
    w = workloads.small(seq_lens=(1500, 333), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=n_q)
    say("graph replay, device lengths, n_q", n_q)
    ref = OracleRun(w)
    steps = 4
    lens = list(w.seq_lens)
    max_len = [L + 64 for L in lens]
    pool, base = _spaced_pool(qk, w, max_len)
    kd, vd = ref.k.cuda(), ref.v.cuda()
    g = qk.calibrate(pool, kd, vd, lens)
    start = [L - steps * n_q for L in lens]
    zero = [0] * w.batch
    qk.append(pool, _seq_rows(kd, w, zero, start), _seq_rows(vd, w, zero, start), g, base, zero, start)
    B, Hq, D = w.batch, w.num_q_heads, w.head_dim
    q_buf = torch.zeros((B, n_q, Hq, D), dtype=torch.bfloat16, device="cuda")
    k_buf = torch.zeros((B * n_q, w.num_kv_heads, D), dtype=torch.bfloat16, device="cuda")
    v_buf = torch.zeros_like(k_buf)
    lens_dev = torch.tensor(start, dtype=torch.int64, device="cuda")
    out_buf = torch.zeros((B, n_q, Hq, D), dtype=torch.float32, device="cuda")
    ws = qk.alloc_workspace(pool, max_len, n_q, Hq)
    torch.cuda.synchronize()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(stream):
        with torch.cuda.graph(graph, stream=stream):
            qk.decode_step_dev_len(pool, g, k_buf, v_buf, q_buf, base, max_len, lens_dev, w.sm_scale, out=out_buf,
                                   workspace=ws)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    gen = torch.Generator().manual_seed(77)
    tol = TOL_REL * ref.vmax()
    for s in range(steps):
        now = [st + (s + 1) * n_q for st in start]
        q_s = torch.randn((B, n_q, Hq, D), generator=gen).to(torch.bfloat16)
        q_buf.copy_(q_s)
        k_buf.copy_(_seq_rows(kd, w, [L - n_q for L in now], now))
        v_buf.copy_(_seq_rows(vd, w, [L - n_q for L in now], now))
        lens_dev.copy_(torch.tensor(now, dtype=torch.int64))
        graph.replay()
        torch.cuda.synchronize()
        exp = oracle.attention(ref.cache, ref.g, workloads.as_u16(q_s), w.seq_base, now, n_q, w.sm_scale)
        err = max_err(out_buf.cpu().numpy(), exp)
        say(f"  step {s} lengths {now}: max err {err:.3e}  tol {tol:.3e}")
        assert err <= tol
    _assert_seq_slots_equal(pool, base, ref, w)
    first = out_buf.clone()
    graph.replay()
    torch.cuda.synchronize()
    assert_same_output(first, out_buf, w, ref.vmax())


@pytest.mark.parametrize("n_q", [2, 6])      # 12 rows: one row tile; 36 rows: the pair kernel
def test_decode_deterministic_and_partial_combine_split(qk, n_q):
    """A second run, and the step as separate partial and combine calls, give the same output:
    bit for bit at one row tile (a fixed block partition), within the attention tolerance in
    the pair kernel (pairs claim blocks as they free up)."""
    w = workloads.small(seq_lens=(5000, 1234), num_kv_heads=4, num_q_heads=24, head_dim=256, n_q=n_q)
    say("determinism", n_q)
    ref = OracleRun(w)
    pool, g, out = gpu_run(w, ref.k, ref.v, ref.q)
    q = ref.q.cuda()
    out2 = qk.decode_attn(pool, g, q, w.seq_base, list(w.seq_lens), w.sm_scale)
    assert_same_output(out, out2, w, ref.vmax())
    ws = qk.alloc_workspace(pool, list(w.seq_lens), w.n_q, w.num_q_heads)
    out3 = torch.empty_like(out)
    qk.decode_attn_partial(pool, g, q, w.seq_base, list(w.seq_lens), w.sm_scale, ws)
    qk.decode_attn_combine(pool, g, out3, list(w.seq_lens), ws)
    torch.cuda.synchronize()
    assert_same_output(out, out3, w, ref.vmax())
    _check_decode(w, ref, out)


@pytest.mark.parametrize("shape", [
    dict(seq_lens=(9000, 3000), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=2),   # 12 rows: one tile
    dict(seq_lens=(9000, 3000), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=4),   # 24 rows: claimed blocks
    dict(seq_lens=(9000, 3000), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=6),   # 36 rows: pair kernel
])
def test_repeat_runs(qk, shape):
    """Five runs of one step: bit-identical for one row tile (a fixed block partition); at two
    row tiles and in the pair kernel, where waves or pairs claim blocks as they free up, every
    run within the attention tolerance of the others and of the oracle."""
    w = workloads.small(**shape)
    say("repeat runs", shape)
    ref = OracleRun(w)
    pool, g, out = gpu_run(w, ref.k, ref.v, ref.q)
    q = ref.q.cuda()
    outs = [out] + [qk.decode_attn(pool, g, q, w.seq_base, list(w.seq_lens), w.sm_scale) for _ in range(4)]
    torch.cuda.synchronize()
    for o in outs[1:]:
        assert_same_output(outs[0], o, w, ref.vmax())
    for o in outs:
        _check_decode(w, ref, o)


def test_split_plan_invariance(qk):
    """Sequence 0 decoded alone and next to a much longer sequence gets a different
    split plan; the results agree to fp32 noise and both pass the oracle check."""
    w = workloads.small(seq_lens=(3000, 60000), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=2)
    say("split invariance")
    ref = OracleRun(w)
    pool, g, out = gpu_run(w, ref.k, ref.v, ref.q)
    q0 = ref.q[:1].cuda()
    g0 = g[:1].contiguous()
    alone = qk.decode_attn(pool, g0, q0, [0], [3000], w.sm_scale)
    torch.cuda.synchronize()
    vmax = ref.vmax()
    assert (alone[0] - out[0]).abs().max().item() <= 1e-5 * vmax
    _check_decode(w, ref, out, sel=[(b, i, h) for b in range(2) for i in range(2) for h in range(0, 12, 5)])


def test_extreme_scores_and_constant_v(qk):
    """Large queries (scores spanning thousands of units: the lazy running-max path
    and its rescale) and V constant per head (output must be that constant)."""
    w = workloads.small(seq_lens=(4000,), num_kv_heads=2, num_q_heads=8, head_dim=256, n_q=3)
    say("extreme scores")
    k = workloads.all_kv_rows(w, "k")
    v = torch.zeros_like(k)
    v[:, 0] = 1.5
    v[:, 1] = -0.75
    q = (workloads.queries(w).float() * 40).to(torch.bfloat16)
    ref = OracleRun(w, k=k, v=v, q=q)
    pool, g, out = gpu_run(w, ref.k, ref.v, ref.q)
    _check_decode(w, ref, out)
    o = out.cpu()
    assert torch.allclose(o[:, :, :4], torch.full_like(o[:, :, :4], 1.5), rtol=0, atol=1e-6)
    assert torch.allclose(o[:, :, 4:], torch.full_like(o[:, :, 4:], -0.75), rtol=0, atol=1e-6)


@pytest.mark.parametrize("n_q", [1, 36])
def test_fp16_probability_floor_long_units(qk, n_q):
    """Probabilities enter the PV product in fp16 against a wave's running reference, so a
    weight below 2^-25 of it rounds to 0. Here every (sequence, KV head) has one key 17.5 nats
    above a flat tail of ~200,000 keys whose V differs from that key's (-1 against +1): each
    tail key's weight rounds to 0 in the wave that holds the dominant key. With one unit per
    (sequence, head) -- 8 sequences x 32 KV heads fill the 256 slots -- that wave would see
    50,000 keys and lose 2.5e-3 of the V range; the planner's 32,768-token unit cap keeps it
    at a quarter of that. The expected output has a closed form (K and V bytes written
    directly): o = (-e^s + N) / (e^s + N) in every element, N the visible tail keys.
    n_q = 1 runs the one-wave kernel, n_q = 36 (36 rows) the pair kernel."""
    B, Hkv, D, L = 8, 32, 128, 200000
    Hq = Hkv
    say("fp16 probability floor, n_q", n_q)
    cap = B * L
    pool = qk.KVPool(Hkv, D, cap, device="cuda")
    base = [b * L for b in range(B)]
    pool.v_codes.fill_(0x22)                 # code 2 in both nibbles: +1.0
    pool.v_scales.fill_(0x38)                # E4M3 1.0
    for b0 in base:
        pool.k_codes[:, b0].fill_(0x22)      # the dominant key: k_hat = 1.0 everywhere
        pool.k_scales[:, b0].fill_(0x38)
        pool.v_codes[:, b0].fill_(0xAA)      # its V: -1.0
    g = torch.ones((B, Hkv, 2), dtype=torch.float32, device="cuda")
    sm = 1.0 / math.sqrt(D)
    c = 1.546875                             # bf16-exact; s = c * D * sm = 17.5 nats
    q = torch.full((B, n_q, Hq, D), c, dtype=torch.bfloat16, device="cuda")
    out = qk.decode_attn(pool, g, q, base, [L] * B, sm)
    torch.cuda.synchronize()
    s = c * D * sm
    got = out.cpu().double()
    worst = 0.0
    for i in range(n_q):
        N = L - n_q + i                      # visible keys 1 .. L - n_q + i
        exp = (-math.exp(s) + N) / (math.exp(s) + N)
        worst = max(worst, (got[:, i] - exp).abs().max().item())
    say(f"  max err {worst:.3e}  tol {TOL_REL:.3e}")
    assert worst <= TOL_REL * 1.0            # max |V_hat| = 1
    del pool


@pytest.mark.parametrize("scale", [-0.0625, 0.0])
def test_nonpositive_softmax_scale(qk, scale):
    """A negative softmax scale (the kernels put its sign into the query fragments and keep
    a positive score factor) and a zero one (uniform weights), on one, two and three row
    tiles."""
    for shape in (dict(seq_lens=(300, 45), num_kv_heads=2, num_q_heads=6, head_dim=256, n_q=1),
                  dict(seq_lens=(700, 129), num_kv_heads=2, num_q_heads=12, head_dim=256, n_q=4),
                  dict(seq_lens=(963,), num_kv_heads=1, num_q_heads=6, head_dim=256, n_q=6)):
        w = workloads.small(**shape)
        say("sm_scale", scale, shape)
        ref = OracleRun(w)
        pool, g, _ = gpu_run(w, ref.k, ref.v, ref.q)
        out = qk.decode_attn(pool, g, ref.q.cuda(), w.seq_base, list(w.seq_lens), scale)
        exp = oracle.attention(ref.cache, ref.g, workloads.as_u16(ref.q), w.seq_base, w.seq_lens, w.n_q, scale)
        err, tol = max_err(out.float().cpu().numpy(), exp), TOL_REL * ref.vmax()
        say(f"  max err {err:.3e}  tol {tol:.3e}")
        assert err <= tol


def test_sequence_at_pool_end_and_zero_kv(qk):
    """A sequence ending exactly at the pool's last slot with a ragged tail (reads past
    the end stay in bounds), all-zero K (uniform weights) and all-zero V."""
    w = workloads.small(seq_lens=(37, 101), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=2)
    say("pool end / zero kv")
    k = torch.zeros((w.capacity, 1, 128), dtype=torch.bfloat16)
    v = workloads.all_kv_rows(w, "v")
    ref = OracleRun(w, k=k, v=v)
    pool, g, out = gpu_run(w, ref.k, ref.v, ref.q)
    _check_decode(w, ref, out)
    ref0 = OracleRun(w, k=workloads.all_kv_rows(w, "k"), v=torch.zeros_like(k))
    pool0, g0, out0 = gpu_run(w, ref0.k, ref0.v, ref0.q)
    assert torch.count_nonzero(out0).item() == 0


def test_workspace_too_small_is_rejected(qk):
    w = workloads.small(seq_lens=(100,), num_kv_heads=1, num_q_heads=4, head_dim=128, n_q=1)
    pool = qk.KVPool(1, 128, 100)
    g = torch.zeros((1, 1, 2), device="cuda")
    q = torch.zeros((1, 1, 4, 128), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(qk.Nvfp4Error) as e:
        qk.decode_attn(pool, g, q, [0], [100], 0.1, workspace=ws)
    assert e.value.code == qk.EWORKSPACE


# ------------------------------------------------------- full-size workloads ------
def _full_step(qk, w, ref):
    """The configuration's timed path: the pool filled up to L - n_q per sequence (the
    max-context workload as its 591,808 rows, then its prefill chunk up to the step's row),
    then one nvfp4_decode_step -- the call the benchmark times, with the workspace size and
    split plan it uses -- storing the step's n_q rows and attending; then the same step
    through nvfp4_decode_step_dev_len with the lengths in device memory (bound = length).
    Returns (pool, g, out_step, out_dev_len)."""
    dev = "cuda"
    pool = qk.KVPool(w.num_kv_heads, w.head_dim, w.capacity, device=dev, kv_format=w.kv_format)
    kd, vd = ref.k.to(dev), ref.v.to(dev)
    lens = list(w.seq_lens)
    g = qk.calibrate(pool, kd, vd, lens)
    zero = [0] * w.batch
    pre = [L - w.n_q for L in lens]
    if w.append_rows:
        L0 = w.capacity - w.append_rows
        qk.append(pool, kd[:L0].contiguous(), vd[:L0].contiguous(), g, [0], [0], [L0])
        qk.append(pool, kd[L0:pre[0]].contiguous(), vd[L0:pre[0]].contiguous(), g, [0], [L0], [pre[0] - L0])
    else:
        qk.append(pool, _seq_rows(kd, w, zero, pre), _seq_rows(vd, w, zero, pre), g, w.seq_base, zero, pre)
    k_step, v_step = _seq_rows(kd, w, pre, lens), _seq_rows(vd, w, pre, lens)
    del kd, vd
    q = ref.q.to(dev)
    ws = qk.alloc_workspace(pool, lens, w.n_q, w.num_q_heads)
    out = qk.decode_step(pool, g, k_step, v_step, q, w.seq_base, lens, w.sm_scale, workspace=ws)
    out_dl = None
    if w.rows <= 128:
        lens_dev = torch.tensor(lens, dtype=torch.int64, device=dev)
        out_dl = qk.decode_step_dev_len(pool, g, k_step, v_step, q, w.seq_base, lens, lens_dev, w.sm_scale,
                                        workspace=ws)
    torch.cuda.synchronize()
    return pool, g, out, out_dl


def _prefill_rows(w):
    return [(b, i, h) for b in range(w.batch) for i in (0, 1, w.n_q // 2, w.n_q - 1) for h in range(w.num_q_heads)]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["tiny", "decode_27b", "mtp_verify", "long_agentic", "append_max_context",
                                  "dflash_verify", "prefill_chunk"])
def test_full_workload_step(qk, name):
    """Every configuration at full size through the timed decode step: the pool bytes (the
    step's own rows included) bit-exact against the oracle's, and every query row's output
    within tolerance (prefill_chunk, 24,576 rows: every head of four query tokens)."""
    w = workloads.get(name)
    say("full workload", name, w.seq_lens, "n_q", w.n_q)
    ref = OracleRun(w)
    say("  oracle quantised; running the GPU step")
    pool, g, out, out_dl = _full_step(qk, w, ref)
    assert np.array_equal(g.cpu().numpy(), ref.g)
    assert_planes_equal(pool, ref.cache)
    say("  planes bit-exact; oracle attention")
    sel = _prefill_rows(w) if name == "prefill_chunk" else None
    _check_decode(w, ref, out, sel=sel)
    if out_dl is not None:
        say("  device-length step")
        _check_decode(w, ref, out_dl, sel=sel)


@pytest.mark.parametrize("nbytes,wg", [(64 * 1024 * 1024 + 48, 1024), ((1 << 31) + (1 << 24) + 16, 4096)])
def test_read_probe_reads_every_word_once(qk, nbytes, wg):
    """The streaming-read probe folds every 32-bit word of the buffer exactly once (the XOR of
    its per-workgroup checksums equals the XOR of the buffer), including a ragged tail and a
    buffer past the 2 GiB window of one raw buffer descriptor."""
    say("read probe", nbytes, "bytes,", wg, "workgroups")
    gen = torch.Generator(device="cuda").manual_seed(5)
    buf = torch.randint(-2 ** 31, 2 ** 31 - 1, (nbytes // 4,), dtype=torch.int32, device="cuda", generator=gen)
    sink = qk.hbm_read_probe(buf, wg)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    exp = np.bitwise_xor.reduce(buf.cpu().numpy().view(np.uint32))
    assert got == exp
    del buf
