#!/usr/bin/env python3
"""NVFP4-KV decode attention benchmark on one MI355X.

One step = one decode layer-step of the hot path for the whole batch:
  quantise-on-append of the n_q new K/V rows per sequence (into NVFP4),
  split-K decode partial pass over the packed cache, combine pass.
Throughput `value` is effective KV GB/s: packed KV bytes read per step / step time
(inputs resident in HBM). The packed cache is rotated over enough copies (>= 1 GiB
in all) that successive steps cannot be served from the 256 MB Infinity Cache.

The K timed steps are captured into one HIP graph (the pages' engine decodes with
exact-batch graphs: knoopx/ninfer page, "Capabilities and limits") and replayed
once between events on the launch stream. Each kernel's average duration comes
from a graph of K launches of that kernel alone, timed the same way.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4-KV decode attention µs/layer-step + effective KV GB/s (% HBM peak)"
HBM_PEAK_GBS = 8000.0
ROTATE_MIN_BYTES = 1 << 30


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# Sources that shape the partial kernel's memory traffic (kernels, shared device code, planner).
DIGEST_SOURCES = ("decode.hip", "decode_pair.hip", "decode_common.h", "quantize.h", "internal.h", "api.cpp")


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in DIGEST_SOURCES:
        h.update(open(os.path.join(ROOT, "quantized_kv_decode_amd", "csrc", f), "rb").read())
    return h.hexdigest()[:16]


def read_traffic(workload: str):
    """HBM bytes per partial-kernel launch from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"decode_partial_{workload}_counters.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            k, v = line.split(":", 1)
            kv[k.strip()] = v.strip()
    if kv.get("kernel_source_digest") != kernel_source_digest():
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, budget_s: float = 12.0):
    """The fp64 oracle timed on the host on a bounded sample of the same workload: the decode
    step (quantise the n_q new K/V rows, then attention for every query row) of the first
    sequence's first KV heads, each over that sequence's whole cache, repeated until about
    budget_s seconds have passed. The rate is the sample's packed KV bytes per step over the
    time per step (the unit of the GPU figure); a second, single-thread leg times the rows
    of one query token of one KV head."""
    import numpy as np
    import oracle
    import workloads
    nthreads = oracle.default_threads()
    b, L = 0, w.seq_lens[0]
    heads = list(range(min(2, w.num_kv_heads)))
    q_all = workloads.as_u16(workloads.queries(w))
    k_rows = workloads.as_u16(workloads.kv_rows(w, "k", b))
    v_rows = workloads.as_u16(workloads.kv_rows(w, "v", b))
    parts = []
    for kh in heads:                         # one single-head cache per sampled KV head
        ku = np.ascontiguousarray(k_rows[:, kh:kh + 1])
        vu = np.ascontiguousarray(v_rows[:, kh:kh + 1])
        g = oracle.calibrate(ku, vu, [L])
        cache = oracle.Cache(1, w.head_dim, L, kv_format=w.kv_format)
        oracle.append(cache, ku, vu, g, [0], [0], [L - w.n_q], nthreads)
        q = np.ascontiguousarray(q_all[b:b + 1, :, kh * w.group:(kh + 1) * w.group])
        kn, vn = np.ascontiguousarray(ku[L - w.n_q:]), np.ascontiguousarray(vu[L - w.n_q:])
        parts.append((cache, g, q, kn, vn))
    del k_rows, v_rows

    def step(cache, g, q, kn, vn, nth, sel=None):
        oracle.append(cache, kn, vn, g, [0], [L - w.n_q], [w.n_q], nth)
        oracle.attention(cache, g, q, [0], [L], w.n_q, w.sm_scale, sel=sel, nthreads=nth)

    steps, t0 = 0, time.perf_counter()
    while True:
        for pt in parts:
            step(*pt, nthreads)
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 1000:
            break
    bytes_per_token = workloads.packed_bytes_per_token_head(w.head_dim, w.kv_format)
    bytes_per_step = len(heads) * L * bytes_per_token
    # one thread: the G rows of the first query token of the first sampled head
    t1 = time.perf_counter()
    step(*parts[0], 1, sel=[(0, 0, h) for h in range(w.group)])
    el1 = time.perf_counter() - t1
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    return {"value": round(bytes_per_step * steps / el / 1e9, 4), "unit": "GB/s", "cores": nthreads,
            "kind": "oracle",
            "sample": f"{steps} decode step(s) of {w.name}'s sequence 0 ({L} tokens), KV heads {heads}: append "
                      f"the {w.n_q} new rows + fp64 attention for all {w.group * w.n_q} query rows of each head "
                      f"over the whole sequence, {el:.1f} s; value = sampled packed KV bytes per step / time",
            "ms_per_step": round(el / steps * 1e3, 3), "threads": nthreads, "nproc": os.cpu_count(),
            "affinity_cpus": affinity,
            "single_thread": {"rows": w.group, "keys_per_row": L - w.n_q + 1, "ms": round(el1 * 1e3, 3),
                              "GBps": round(L * bytes_per_token / el1 / 1e9 * w.group / (w.group * w.n_q), 4)},
            "cpu_model": cpu_model()}


def hbm_probe(dev, nbytes: int = 1 << 30):
    """Best plain streaming read rate (GB/s) over a few launch sizes of the library's read
    probe, each timed over 10 launches between events."""
    import torch
    import quantized_kv_decode_amd as qk
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.empty(16384, dtype=torch.int32, device=dev)
    s = torch.cuda.current_stream()
    best, rates = 0.0, {}
    for wg in (256, 512, 768, 1024, 1536, 2048, 4096, 8192):
        for _ in range(3):
            qk.hbm_read_probe(buf, wg, sink)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(s)
        for _ in range(10):
            qk.hbm_read_probe(buf, wg, sink)
        e1.record(s)
        e1.synchronize()
        gbps = nbytes * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
        rates[wg] = round(gbps, 1)
        best = max(best, gbps)
    del buf, sink
    return best, rates


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=int(os.environ.get("WORLD_SIZE", "1")))
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="long_agentic")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="run one plain device copy of this many MiB (read + write) before timing, as a "
                         "reference dispatch of known size for HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        return 2

    import torch
    import quantized_kv_decode_amd as qk
    import workloads

    qk.load_library()
    w = workloads.get(args.workload)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    K, W = args.steps, args.warmup

    # ---- resident inputs: one calibrated, filled pool, then rotation copies
    log(f"workload {w.name}: {w.description}")
    pool0 = qk.KVPool(w.num_kv_heads, w.head_dim, w.capacity, device=dev, kv_format=w.kv_format)
    g = torch.empty((w.batch, w.num_kv_heads, 2), dtype=torch.float32, device=dev)
    kdev, vdev = [], []
    for b in range(w.batch):                                   # upload per sequence
        kdev.append(workloads.kv_rows(w, "k", b).to(dev))
        vdev.append(workloads.kv_rows(w, "v", b).to(dev))
    kall, vall = torch.cat(kdev), torch.cat(vdev)
    del kdev, vdev
    qk.calibrate(pool0, kall, vall, list(w.seq_lens), out=g)
    if w.append_rows:                                          # prefill chunk appended on its own
        L0 = w.capacity - w.append_rows
        qk.append(pool0, kall[:L0].contiguous(), vall[:L0].contiguous(), g, [0], [0], [L0])
    else:
        qk.append(pool0, kall, vall, g, w.seq_base, [0] * w.batch, list(w.seq_lens))
    rows = torch.cat([torch.arange(w.seq_base[b] + w.seq_lens[b] - w.n_q, w.seq_base[b] + w.seq_lens[b])
                      for b in range(w.batch)]).to(dev)
    k_step, v_step = kall[rows].contiguous(), vall[rows].contiguous()
    chunk = None
    if w.append_rows:
        chunk = (kall[w.capacity - w.append_rows:].contiguous(), vall[w.capacity - w.append_rows:].contiguous())
    del kall, vall
    q = workloads.queries(w).to(dev)
    if chunk is not None:
        qk.append(pool0, chunk[0], chunk[1], g, [0], [w.capacity - w.append_rows], [w.append_rows])
    R = max(1, math.ceil(ROTATE_MIN_BYTES / pool0.nbytes)) if pool0.nbytes < (256 << 20) * 2 else 1
    pools = [pool0] + [qk.KVPool.from_planes(pool0.k_codes.clone(), pool0.k_scales.clone(), pool0.v_codes.clone(),
                                             pool0.v_scales.clone()) for _ in range(R - 1)]
    ws = qk.alloc_workspace(pool0, list(w.seq_lens), w.n_q, w.num_q_heads, dev)
    out = torch.empty((w.batch, w.n_q, w.num_q_heads, w.head_dim), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"cache {pool0.nbytes / 1e6:.1f} MB x {R} rotation copies; workspace {ws.numel() / 1e6:.2f} MB")

    wp = [L - w.n_q for L in w.seq_lens]
    nq = [w.n_q] * w.batch
    seq_lens = list(w.seq_lens)

    def k_append(p):
        qk.append(p, k_step, v_step, g, w.seq_base, wp, nq)

    def k_partial(p):
        qk.decode_attn_partial(p, g, q, w.seq_base, seq_lens, w.sm_scale, ws)

    def k_combine(p):
        qk.decode_attn_combine(p, g, out, seq_lens, ws)

    def k_decode_step(p):
        # one decode step: the decode kernel stores the step's n_q rows per sequence itself
        # (fused append), then the combine kernel: two launches
        qk.decode_step(p, g, k_step, v_step, q, w.seq_base, seq_lens, w.sm_scale, out=out, workspace=ws)

    def step(i):
        k_decode_step(pools[i % R])

    if args.copy_calibration_mb:
        n = args.copy_calibration_mb << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {n} bytes read + {n} bytes written in one copy dispatch")
        del src, dst

    # ---- warmup (eager) and the reference output of the eager path
    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    def capture(fn_list, n):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(n):
                    for fn in fn_list:
                        fn(pools[i % R])
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        return graph

    def time_graph(graph, reps=1):
        s = torch.cuda.current_stream()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        # untimed replays first: graph upload, and at least ~30 ms of the same work so that the
        # timed replay does not start on clocks that dropped while the host captured graphs
        e0.record(s)
        graph.replay()
        e1.record(s)
        e1.synchronize()
        for _ in range(min(50, int(30.0 / max(e0.elapsed_time(e1), 1e-3)))):
            graph.replay()
        torch.cuda.synchronize()
        e0.record(s)
        for _ in range(reps):
            graph.replay()
        e1.record(s)
        e1.synchronize()
        return e0.elapsed_time(e1)                            # ms

    g_step = capture([k_decode_step], K)
    g_part = capture([k_partial], K)
    g_comb = capture([k_combine], K)
    g_app = capture([k_append], K)

    # ---- timed region: exactly K steps
    torch.cuda.synchronize()
    ms_total = time_graph(g_step)
    ms_step = ms_total / K
    ms_part = time_graph(g_part) / K
    ms_comb = time_graph(g_comb) / K
    ms_app = time_graph(g_app) / K
    chunk_res = None
    if chunk is not None:
        # the prefill-chunk append of this workload, reported on its own
        def k_chunk(p):
            qk.append(p, chunk[0], chunk[1], g, [0], [w.capacity - w.append_rows], [w.append_rows])
        ms_chunk = time_graph(capture([k_chunk], K)) / K
        rd = w.append_rows * w.num_kv_heads * w.head_dim * 2 * 2
        wr = w.append_rows * w.num_kv_heads * (w.head_dim // 2 + w.head_dim // 16) * 2
        chunk_res = {"rows": w.append_rows, "us": round(ms_chunk * 1e3, 3), "bytes_read": rd, "bytes_written": wr,
                     "GBps": round((rd + wr) / (ms_chunk * 1e-3) / 1e9, 2)}
    # spread of the step over repeated replays of the same graph (after the timed one)
    reps = [time_graph(g_step) / K * 1e3 for _ in range(7)]
    qs = sorted(reps)
    spread = {"p10": round(qs[0], 3), "p50": round(qs[3], 3), "p90": round(qs[6], 3), "replays": 7}
    # plain stream launches of the same K steps (no graph), between events
    s0 = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for i in range(W):
        step(i)
    e0.record(s0)
    for i in range(K):
        step(i)
    e1.record(s0)
    e1.synchronize()
    eager_us = e0.elapsed_time(e1) / K * 1e3
    # with the cache allowed to stay in the 256 MB Infinity Cache (no rotation): labelled apart
    warm_us = None
    if R > 1:
        sw = torch.cuda.Stream()
        sw.wait_stream(torch.cuda.current_stream())
        g_warm = torch.cuda.CUDAGraph()
        with torch.cuda.stream(sw):
            with torch.cuda.graph(g_warm, stream=sw):
                for i in range(K):
                    k_decode_step(pools[0])
        torch.cuda.current_stream().wait_stream(sw)
        torch.cuda.synchronize()
        warm_us = time_graph(g_warm) / K * 1e3
    # the same step with the lengths in device memory (nvfp4_decode_step_dev_len, bound = length),
    # which one captured graph can replay across steps; reported next to the main line
    lens_dev = torch.tensor(seq_lens, dtype=torch.int64, device=dev)
    out_dl = torch.empty_like(out)

    def k_step_dev_len(p):
        qk.decode_step_dev_len(p, g, k_step, v_step, q, w.seq_base, seq_lens, lens_dev, w.sm_scale, out=out_dl,
                               workspace=ws)
    # (above 128 query rows per KV head that step does not store its rows itself: not timed)
    dev_len = w.group * w.n_q <= 128
    ms_dl = time_graph(capture([k_step_dev_len], K)) / K if dev_len else None
    out_graph = out.clone()
    step(0)                                                    # eager step on copy 0: same result
    torch.cuda.synchronize()
    # the same step replayed from the graph and run eagerly: identical bits where the kernels'
    # block partition is fixed; at two row tiles (waves claim blocks as they free up) equal to
    # rounding (observed: 3e-4 of the output range at most)
    assert (out - out_graph).abs().max().item() <= 2e-3 * out.abs().max().item(), "graph replay and eager step disagree"
    # device-planned splits may differ from the host's: the same result up to rounding (fp32
    # summation order, and the fp16 rounding of probabilities against each wave's reference)
    if dev_len:
        assert (out_dl - out).abs().max().item() <= 2e-3 * out.abs().max().item(), "device-length step disagrees"

    log("read probe")
    achievable, probe_rates = hbm_probe(dev)
    kv = w.kv_bytes
    achieved = kv / (ms_part * 1e-3) / 1e9
    traffic = read_traffic(w.name)
    res = {
        "metric": METRIC,
        "value": round(kv / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 6),
        "us_per_layer_step": round(ms_step * 1e3, 3),
        "pct_hbm_peak": round(kv / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS * 100, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": w.name,
            "batch": w.batch,
            "seq_lens": list(w.seq_lens),
            "num_kv_heads": w.num_kv_heads,
            "num_q_heads": w.num_q_heads,
            "head_dim": w.head_dim,
            "n_q": w.n_q,
            "kv_format": ("nvfp4 (e2m1 codes + e4m3 group-16 scales + fp32 per-(seq, kv head) scale)"
                          if w.kv_format == "nvfp4" else
                          "k8v4 (K: e4m3 codes + fp32 row scale; V: nvfp4 as above)"),
            "kv_bytes_per_step": kv,
            "rotation_copies": R,
            "timing": "one HIP-graph replay of K steps between events",
            "step": "decode step (nvfp4_decode_step): split-K partial with the n_q-row append fused in, then combine",
        },
        "kernels_us": {"append": round(ms_app * 1e3, 3), "decode_partial": round(ms_part * 1e3, 3),
                       "decode_combine": round(ms_comb * 1e3, 3)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "decode_partial", "algorithmic_bytes_per_launch": kv},
    }
    step_gbps = kv / (ms_step * 1e-3) / 1e9
    res["achievable"] = {"GBps": round(achievable, 1), "step_frac": round(step_gbps / achievable, 4),
                         "partial_frac": round(achieved / achievable, 4),
                         "probe": "plain streaming read of 1 GiB, 16-byte non-temporal loads (nvfp4_hbm_read_probe), best of "
                                  "these workgroup counts", "by_workgroups": probe_rates}
    res["device_lengths_step_us"] = round(ms_dl * 1e3, 3) if dev_len else None
    res["step_us_spread"] = spread
    res["stream_launch_step_us"] = round(eager_us, 3)
    res["warm_infinity_cache_step_us"] = round(warm_us, 3) if warm_us is not None else None
    # attention arithmetic of the step (QK^T and PV over the visible keys, 2 flops per
    # multiply-add), against MI355X's dense fp16 matrix peak: the bound for long query chunks
    res["attention_tflops"] = round(w.flops / (ms_step * 1e-3) / 1e12, 2)
    res["attention_flops_per_step"] = w.flops
    if chunk_res is not None:
        res["append_chunk"] = chunk_res
    if not args.no_cpu_baseline:
        log("timing the CPU oracle")
        res["cpu_baseline"] = cpu_baseline(w, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
