"""Oracle: which token rows a context-parallel rank holds.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).

Sources:
* "04 · Megatron-LM 实现" (Megatron CP integration page), section 1.1 "pretrain:
  zigzag 切分": the sequence is viewed as 2·cp equal chunks and rank r keeps chunk r
  and chunk 2·cp−1−r, in that order, each chunk's rows in ascending order; the
  sequence length must be divisible by 2·cp.
* same page, section 1.2 (packed THD): the split is done inside every
  sub-sequence ("per-sub-sequence zigzag"), and section 5 (RoPE under zigzag): for
  each sub-sequence the rank takes the front slice [r·seg, (r+1)·seg) and the
  mirrored back slice [len−(r+1)·seg, len−r·seg), seg = len/(2·cp), concatenated.
* "Context Parallelism (CP)" page, section 4: with cp=2 the four chunks go
  (chunk0, chunk3) to rank 0 and (chunk1, chunk2) to rank 1.
* "推理系统基础设施（二）：Sequence Parallelism + Ring Attention" (ring-attention
  page), section 5: the interleaved assignment [0, 4, 8, ...], [1, 5, 9, ...] for four
  ranks; "Context Parallelism (CP)" page, sections 2.4 and 4, names this striped
  split as the other static balancer of the causal task graph.  Reading: the
  interleave is per token (rank r holds the tokens whose index is r modulo cp), as
  in the Striped Attention paper the CP page cites.

Pins: tests/test_oracle_partition.py (the cp=2 assignment and the cp=4 interleave
printed on the pages, permutation / balance invariants and closed-form pair counts,
a second formulation by reshaping each document).
"""
from __future__ import annotations

import numpy as np


def zigzag_indices(seq_len: int, cp: int, rank: int) -> np.ndarray:
    """Global row indices held by ``rank``: chunk ``rank`` then chunk ``2cp-1-rank``.

    Raises ValueError unless seq_len % (2*cp) == 0 and 0 <= rank < cp (the
    alignment assertion of the Megatron page, section 1.1)."""
    if cp < 1 or not (0 <= rank < cp):
        raise ValueError("rank out of range")
    if seq_len % (2 * cp) != 0:
        raise ValueError("sequence length must be divisible by 2*cp")
    chunk = seq_len // (2 * cp)
    rows = []
    for c in (rank, 2 * cp - 1 - rank):
        for t in range(chunk):
            rows.append(c * chunk + t)
    return np.asarray(rows, dtype=np.int64)


def striped_indices(seq_len: int, cp: int, rank: int) -> np.ndarray:
    """Global row indices held by ``rank`` under the striped (interleaved) split:
    rank, rank + cp, rank + 2cp, ...  The length must be divisible by cp."""
    if cp < 1 or not (0 <= rank < cp):
        raise ValueError("rank out of range")
    if seq_len % cp != 0:
        raise ValueError("sequence length must be divisible by cp")
    rows = []
    t = rank
    while t < seq_len:
        rows.append(t)
        t += cp
    return np.asarray(rows, dtype=np.int64)


def thd_indices(cu_seqlens, cp: int, rank: int) -> np.ndarray:
    """Per-document zigzag over a packed stream with boundaries ``cu_seqlens``.

    Documents are visited in order; for document k of length L starting at cu[k],
    with seg = L/(2cp): rows cu[k]+[r*seg, (r+1)*seg) then cu[k]+[L-(r+1)*seg, L-r*seg).
    Every length must be divisible by 2*cp."""
    cu = [int(x) for x in cu_seqlens]
    if cp < 1 or not (0 <= rank < cp):
        raise ValueError("rank out of range")
    if cu[0] != 0 or any(b < a for a, b in zip(cu, cu[1:])):
        raise ValueError("cu_seqlens must start at 0 and be non-decreasing")
    rows = []
    for k in range(len(cu) - 1):
        start, length = cu[k], cu[k + 1] - cu[k]
        if length % (2 * cp) != 0:
            raise ValueError("every sub-sequence length must be divisible by 2*cp")
        seg = length // (2 * cp)
        for t in range(rank * seg, (rank + 1) * seg):
            rows.append(start + t)
        for t in range(length - (rank + 1) * seg, length - rank * seg):
            rows.append(start + t)
    return np.asarray(rows, dtype=np.int64)


def thd_doc_ids(cu_seqlens, rows) -> np.ndarray:
    """Document id of each global row (the per-token sequence id of a packed batch)."""
    cu = [int(x) for x in cu_seqlens]
    out = np.empty(len(rows), dtype=np.int64)
    for n, row in enumerate(rows):
        k = 0
        while not (cu[k] <= row < cu[k + 1]):
            k += 1
        out[n] = k
    return out
