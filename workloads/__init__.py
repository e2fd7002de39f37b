"""Seeded synthetic inputs for the five workloads of one context-parallel rank's share.

This module is shared by the tests, the benchmark and the oracle's callers.  It
holds input recipes only: shapes, seeds, random tensors and the packed-sequence
length mix.  It contains none of the attention arithmetic, no partitioning and no
masking, so neither side of a parity check can borrow the other's logic from it.

Workloads (each one rank's share; B = 1 so [T, H, d] token-major everywhere):

* ``tiny``    S=512, cp=2 zigzag (4 chunks of 128), H=1, d=64, fp32, both ranks.
* ``s8k``     S=8192, cp=4 zigzag (8 chunks of 1024), H=8, d=128, bf16, ranks 0..3,
              KV as the 4 owners' segments in ring order.
* ``s128k``   S=131072, cp=8 zigzag (16 chunks of 8192), Hq=32 over Hkv=8 (GQA),
              d=128, bf16, rank 0, KV as 16 chunk segments.
* ``thd64k``  packed variable-length stream of 65536 tokens, lengths lognormal
              (median 2048, sigma 1) clipped to [128, 16384] and rounded to a
              multiple of 8; per-document zigzag with cp=4, rank 1; H=16, d=128, bf16.
* ``bwd8k``   the ``s8k`` shape plus an upstream gradient G ~ N(0,1) bf16.

The long-context shapes follow the 128K worked example of the "Context Parallelism
(CP)" page (section 8); the packed mix stands in for the long-tailed corpus lengths
that page's section 5 describes (no dataset is read).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

__all__ = ["Workload", "WORKLOADS", "randn", "thd_lengths", "cu_seqlens_from_lengths",
           "full_qkv", "upstream_grad"]


@dataclass(frozen=True)
class Workload:
    name: str
    seq: int            # total tokens of the (packed) sequence
    cp: int             # context-parallel size
    hq: int
    hkv: int
    d: int
    dtype: str          # "f32" or "bf16"
    seed: int
    ranks: tuple        # which rank shares are exercised
    kv_granularity: str  # "owner" (one segment per owning rank) or "chunk"
    packed: bool = False
    grad_seed: int | None = None
    notes: str = ""


WORKLOADS = {
    "tiny": Workload("tiny", 512, 2, 1, 1, 64, "f32", 1, (0, 1), "chunk"),
    "s8k": Workload("s8k", 8192, 4, 8, 8, 128, "bf16", 2, (0, 1, 2, 3), "owner"),
    "s128k": Workload("s128k", 131072, 8, 32, 8, 128, "bf16", 3, (0,), "chunk"),
    "thd64k": Workload("thd64k", 65536, 4, 16, 16, 128, "bf16", 4, (1,), "owner", packed=True),
    "bwd8k": Workload("bwd8k", 8192, 4, 8, 8, 128, "bf16", 2, (0, 1, 2, 3), "owner", grad_seed=5),
}


def _torch_dtype(dtype: str):
    return {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]


def randn(shape, seed: int, dtype: str = "bf16", stream: int = 0) -> torch.Tensor:
    """iid N(0,1) CPU tensor drawn in float32 from a seeded generator, then stored in
    ``dtype`` (bf16 by round-to-nearest-even).  ``stream`` separates Q, K, V, G."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed) * 1000003 + int(stream))
    x = torch.randn(tuple(shape), generator=g, dtype=torch.float32)
    return x.to(_torch_dtype(dtype))


def full_qkv(w: Workload, seq: int | None = None):
    """Full-sequence Q [S,Hq,d], K [S,Hkv,d], V [S,Hkv,d] on the CPU."""
    s = w.seq if seq is None else seq
    q = randn((s, w.hq, w.d), w.seed, w.dtype, 0)
    k = randn((s, w.hkv, w.d), w.seed, w.dtype, 1)
    v = randn((s, w.hkv, w.d), w.seed, w.dtype, 2)
    return q, k, v


def upstream_grad(w: Workload, rows: int) -> torch.Tensor:
    """Upstream gradient G [rows, Hq, d] for one rank's local queries."""
    assert w.grad_seed is not None
    return randn((rows, w.hq, w.d), w.grad_seed, w.dtype, 3)


def thd_lengths(seed: int, total: int = 65536, lo: int = 128, hi: int = 16384,
                align: int = 8, median: float = 2048.0, sigma: float = 1.0):
    """Packed-sequence length mix.

    Lengths are lognormal(ln median, sigma), clipped to [lo, hi] and rounded to the
    nearest multiple of ``align``; documents are appended until ``total`` is reached,
    the last one truncated to fit; a truncated tail shorter than ``lo`` is folded into
    the previous document (the only way a length can leave [lo, hi]).
    """
    rng = np.random.default_rng(seed)
    out = []
    acc = 0
    while acc < total:
        x = float(rng.lognormal(math.log(median), sigma))
        x = min(max(x, lo), hi)
        ell = align * int(math.floor(x / align + 0.5))
        ell = min(ell, total - acc)
        out.append(ell)
        acc += ell
    if len(out) > 1 and out[-1] < lo:
        tail = out.pop()
        out[-1] += tail
    return out


def cu_seqlens_from_lengths(lengths) -> np.ndarray:
    """Document boundaries [n+1] int32 from a list of lengths (running sum from 0)."""
    cu = np.zeros(len(lengths) + 1, dtype=np.int64)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu.astype(np.int32)
