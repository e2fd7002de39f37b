"""Oracle: rotary position embedding of a rank's rows at their true positions.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  float64 throughout.

Sources:
* "04 · Megatron-LM 实现" (Megatron CP integration page), section 5: rotary
  embedding depends on absolute positions, so after the split the positions (and
  the frequency table) must be cut exactly like the tokens: the zigzag chunk pair
  [r, 2cp−1−r] of the sequence; for packed documents, per document the front slice
  freqs[r·seg, (r+1)·seg) and the mirrored slice freqs[L−(r+1)·seg, L−r·seg)
  concatenated.  Same page, checklist: a token split and a RoPE split that disagree
  give a silently wrong loss.
* "Context Parallelism (CP)" page, section 5: in a packed stream the position ids
  restart at 0 in every document.

Readings (the rotation itself is not written on the pages): the standard rotary
embedding, angle θ_{p,i} = p · base^(−2i/d) for i = 0 .. d/2−1 (base 10000 unless
given), applied to each head of a row.  Two pairings are common: ``interleaved=False``
rotates (x_i, x_{i+d/2}) — the "rotate half" layout Megatron uses by default — and
``interleaved=True`` rotates (x_{2i}, x_{2i+1}).  Each pair (a, b) becomes
(a cos θ − b sin θ, b cos θ + a sin θ).

Pins: tests/test_oracle_rope.py (hand-computed rotations, the complex-number form,
the relative-position property, norm preservation, and the pages' slicing rules:
rotating then partitioning equals partitioning then rotating at the kept positions).
"""
from __future__ import annotations

import numpy as np


def inv_freq(d: int, base: float = 10000.0) -> np.ndarray:
    """θ_i = base^(−2i/d), i = 0 .. d/2−1."""
    if d % 2 != 0:
        raise ValueError("head dim must be even")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / d)


def angles(pos, d: int, base: float = 10000.0) -> np.ndarray:
    """[len(pos), d/2] rotation angles p · θ_i."""
    return np.outer(np.asarray(pos, dtype=np.float64), inv_freq(d, base))


def apply_rope(x, pos, base: float = 10000.0, interleaved: bool = False) -> np.ndarray:
    """Rotate every head of row t of x [T, H, d] by the angles of position pos[t]."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)
        x = x.to(torch.float64).numpy()
    x = np.asarray(x, dtype=np.float64)
    t, h, d = x.shape
    ang = angles(pos, d, base)[:, None, :]   # [T, 1, d/2]
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty_like(x)
    if interleaved:
        a, b = x[..., 0::2], x[..., 1::2]
        out[..., 0::2] = a * c - b * s
        out[..., 1::2] = b * c + a * s
    else:
        a, b = x[..., : d // 2], x[..., d // 2:]
        out[..., : d // 2] = a * c - b * s
        out[..., d // 2:] = b * c + a * s
    return out


def thd_positions(cu_seqlens, rows) -> np.ndarray:
    """Position of each global row inside its own document (ids restart per document)."""
    cu = [int(x) for x in cu_seqlens]
    out = np.empty(len(rows), dtype=np.int64)
    for n, row in enumerate(rows):
        k = 0
        while not (cu[k] <= row < cu[k + 1]):
            k += 1
        out[n] = row - cu[k]
    return out
