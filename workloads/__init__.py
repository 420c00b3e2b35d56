"""Seeded synthetic inputs for NVFP4-KV decode attention.

This module only draws random numbers and describes workload shapes. It holds
none of the method's arithmetic (no quantisation, no attention), so the CPU
oracle and the HIP path can both take their inputs from here without sharing
any implementation.

Shapes and distributions follow the five workloads the pages motivate: the
long-context agentic sessions (gzenz/ninfer page, "Fork changes vs upstream":
555k-token contexts with 3 concurrent sessions, 330k-470k verified sessions,
600k at one session), MTP verification with 1 + 5 drafts (knoopx/ninfer page,
"Capabilities and limits"), batched decode of 1-8 requests, and the NVFP4 KV
cache itself (gzenz/ninfer page, "Context and model").

Every tensor is generated in fixed chunks of ``CHUNK_ROWS`` rows, each chunk
from its own seeded ``torch.Generator``. Any row range of any tensor is
therefore reproducible on its own, whoever asks for it and in whatever order.

Seeds: for the workload with index k, Q uses 1000k+1, K 1000k+2, V 1000k+3
and the outlier-channel choice 1000k+4.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK_ROWS = 4096

# Bytes per token per KV head of the packed layout. NVFP4: K and V each carry D/2 code
# bytes (two E2M1 codes per byte) and D/16 E4M3 scale bytes. K8V4: K carries D E4M3 code
# bytes and one fp32 row scale, V is NVFP4.
def packed_bytes_per_token_head(head_dim: int, kv_format: str = "nvfp4") -> int:
    v = head_dim // 2 + head_dim // 16
    if kv_format == "k8v4":
        return head_dim + 4 + v
    return 2 * v


@dataclass(frozen=True)
class Workload:
    name: str
    index: int                    # 1-based; selects the seed family
    seq_lens: tuple               # context length per sequence (includes the n_q query tokens)
    num_kv_heads: int
    num_q_heads: int
    head_dim: int
    n_q: int                      # query tokens per sequence (1 + drafts), causal among themselves
    v_dist: str = "normal"        # "normal" or "laplace"
    outlier_frac: float = 0.0     # fraction of channels scaled by outlier_gain in K and V
    outlier_gain: float = 20.0
    append_rows: int = 0          # size of the separately timed prefill-chunk append (0: none)
    description: str = ""
    kv_format: str = "nvfp4"      # "nvfp4", or "k8v4" (row-scaled FP8 E4M3 K, NVFP4 V)

    # ---- derived shapes -------------------------------------------------
    @property
    def batch(self) -> int:
        return len(self.seq_lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def rows(self) -> int:
        """Query rows sharing one KV head: GQA group x query tokens."""
        return self.group * self.n_q

    @property
    def sm_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def capacity(self) -> int:
        """Token slots per head plane when sequences are packed back to back."""
        return int(sum(self.seq_lens))

    @property
    def seq_base(self) -> list:
        base, out = 0, []
        for L in self.seq_lens:
            out.append(base)
            base += L
        return out

    @property
    def n_outlier_channels(self) -> int:
        return int(round(self.outlier_frac * self.head_dim))

    # ---- algorithmic cost -------------------------------------------------
    @property
    def kv_bytes(self) -> int:
        """Packed K+V bytes one decode step must read (codes + E4M3 scales)."""
        return self.capacity * self.num_kv_heads * packed_bytes_per_token_head(self.head_dim, self.kv_format)

    @property
    def visible_keys(self) -> int:
        """Sum over (sequence, query token) of keys visible under the bottom-right causal mask."""
        tot = 0
        for L in self.seq_lens:
            for i in range(self.n_q):
                tot += L - self.n_q + i + 1
        return tot

    @property
    def flops(self) -> int:
        """QK^T plus PV multiply-adds, 2 flops each, over the visible keys of every query head."""
        return 4 * self.num_q_heads * self.head_dim * self.visible_keys


WORKLOADS = {
    "tiny": Workload(
        "tiny", 1, (512,), 1, 4, 128, 1,
        description="1 sequence x 512, 1 KV head, 4 query heads, head_dim 128, 1 query token"),
    "decode_27b": Workload(
        "decode_27b", 2, (32768, 32768), 4, 24, 256, 1,
        description="27B-style decode: batch 2 x 32768, 4 KV / 24 query heads, head_dim 256, 1 query token"),
    "mtp_verify": Workload(
        "mtp_verify", 3, (131072,), 4, 24, 256, 6, outlier_frac=0.02,
        description="MTP verify: 1 x 131072, 6 query tokens (1 + 5 drafts) causal, 2% channels x20"),
    "long_agentic": Workload(
        "long_agentic", 4, (330000, 400000, 470000), 4, 24, 256, 4, v_dist="laplace",
        description="3 ragged sessions 330k/400k/470k, 4 query tokens (1 + 3 drafts), V ~ Laplace(0,1)"),
    "append_max_context": Workload(
        "append_max_context", 5, (600000,), 4, 24, 256, 1, append_rows=8192,
        description="append an 8192-row prefill chunk into a 600000-token cache, then decode over all 600000"),
    # not one of the five configurations: a wide draft window (DFlash-style, 1 + 15 drafts),
    # 96 query rows per KV head, which the decode path serves as three 32-row chunks side by side
    "dflash_verify": Workload(
        "dflash_verify", 6, (131072,), 4, 24, 256, 16, outlier_frac=0.02,
        description="wide draft verify: 1 x 131072, 16 query tokens (1 + 15 drafts) causal, 2% channels x20"),
    # not one of the five configurations: chunked prefill, a 1024-token chunk appended and
    # attending (causally among itself) over a 32768-token context, 6144 query rows per KV head
    "prefill_chunk": Workload(
        "prefill_chunk", 7, (32768,), 4, 24, 256, 1024,
        description="chunked prefill: a 1024-token chunk ending a 32768-token context, causal, 4 KV / 24 query heads"),
}

ORDER = ["tiny", "decode_27b", "mtp_verify", "long_agentic", "append_max_context"]

# The same five configurations stored as K8V4 (8-bit K, NVFP4 V): same seeds, so the same
# bf16 inputs as their NVFP4 versions.
for _n in ORDER:
    _w = WORKLOADS[_n]
    WORKLOADS[_n + "_k8v4"] = Workload(
        _n + "_k8v4", _w.index, _w.seq_lens, _w.num_kv_heads, _w.num_q_heads, _w.head_dim, _w.n_q,
        v_dist=_w.v_dist, outlier_frac=_w.outlier_frac, outlier_gain=_w.outlier_gain,
        append_rows=_w.append_rows, description=_w.description + "; K8V4 (row-scaled FP8 K, NVFP4 V)",
        kv_format="k8v4")
ORDER_K8V4 = [n + "_k8v4" for n in ORDER]


def get(name: str) -> Workload:
    return WORKLOADS[name]


# ---- generators -------------------------------------------------------------
_TENSOR_ID = {"q": 1, "k": 2, "v": 3, "outlier": 4}


def _seed(w: Workload, tensor: str) -> int:
    return 1000 * w.index + _TENSOR_ID[tensor]


def _chunk_generator(base_seed: int, seq: int, chunk: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(base_seed * 1_000_000 + seq * 10_000 + chunk)
    return g


def _draw(dist: str, shape, gen: torch.Generator) -> torch.Tensor:
    if dist == "normal":
        return torch.randn(shape, generator=gen, dtype=torch.float32)
    if dist == "laplace":
        # Laplace(0, 1) by inverse CDF from a uniform drawn in float64.
        u = torch.rand(shape, generator=gen, dtype=torch.float64).clamp_(min=2.0 ** -53)
        c = u - 0.5
        x = -torch.sign(c) * torch.log1p(-2.0 * c.abs())
        return x.to(torch.float32)
    raise ValueError(dist)


def outlier_channels(w: Workload, which: str) -> torch.Tensor:
    """Channels scaled by ``outlier_gain``: [num_kv_heads, n_outlier_channels] int64.

    K and V get independent channel sets (one seeded permutation per head).
    """
    n = w.n_outlier_channels
    g = torch.Generator(device="cpu")
    g.manual_seed(_seed(w, "outlier") * 10 + (0 if which == "k" else 1))
    out = torch.empty((w.num_kv_heads, n), dtype=torch.int64)
    for h in range(w.num_kv_heads):
        out[h] = torch.randperm(w.head_dim, generator=g)[:n]
    return out


def kv_rows(w: Workload, which: str, seq: int, start: int = 0, stop: int | None = None) -> torch.Tensor:
    """bf16 K or V rows [stop-start, num_kv_heads, head_dim] of sequence ``seq`` (CPU)."""
    assert which in ("k", "v")
    L = w.seq_lens[seq]
    stop = L if stop is None else stop
    assert 0 <= start <= stop <= L
    dist = "normal" if which == "k" else w.v_dist
    out = torch.empty((stop - start, w.num_kv_heads, w.head_dim), dtype=torch.bfloat16)
    base = _seed(w, which)
    chans = outlier_channels(w, which) if w.n_outlier_channels else None
    c0, c1 = start // CHUNK_ROWS, (stop - 1) // CHUNK_ROWS if stop > start else -1
    for c in range(c0, c1 + 1):
        r0 = c * CHUNK_ROWS
        r1 = min(r0 + CHUNK_ROWS, L)
        x = _draw(dist, (r1 - r0, w.num_kv_heads, w.head_dim), _chunk_generator(base, seq, c))
        if chans is not None:
            for h in range(w.num_kv_heads):
                x[:, h, chans[h]] *= w.outlier_gain
        lo, hi = max(r0, start), min(r1, stop)
        out[lo - start:hi - start] = x[lo - r0:hi - r0].to(torch.bfloat16)
    return out


def all_kv_rows(w: Workload, which: str) -> torch.Tensor:
    """Rows of every sequence concatenated: [capacity, num_kv_heads, head_dim] bf16."""
    return torch.cat([kv_rows(w, which, b) for b in range(w.batch)], dim=0)


def queries(w: Workload) -> torch.Tensor:
    """bf16 queries [batch, n_q, num_q_heads, head_dim] ~ N(0, 1)."""
    g = _chunk_generator(_seed(w, "q"), 0, 0)
    return torch.randn((w.batch, w.n_q, w.num_q_heads, w.head_dim), generator=g).to(torch.bfloat16)


def as_u16(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU bf16 tensor as a numpy uint16 array (no copy)."""
    assert t.dtype == torch.bfloat16 and t.device.type == "cpu"
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def from_u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)


def small(name: str = "small", seq_lens=(200, 77), num_kv_heads=2, num_q_heads=6, head_dim=256,
          n_q=3, v_dist="normal", outlier_frac=0.0, index=9, kv_format="nvfp4") -> Workload:
    """Ad-hoc workload for parity tests: several tiles, a ragged tail, same generators."""
    return Workload(name, index, tuple(seq_lens), num_kv_heads, num_q_heads, head_dim, n_q,
                    v_dist=v_dist, outlier_frac=outlier_frac, kv_format=kv_format)
