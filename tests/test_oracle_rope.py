"""Pins for the rotary-embedding oracle (CPU only).

What fixes the answers:
* hand-computed rotations: a unit vector on one component of a pair at position p
  becomes (cos pθ, sin pθ) on that pair, with the textbook values of cos and sin at
  1, 2 and 3 radians typed in below;
* the complex-number form of the rotation, (a + ib) e^{iθ}, as a second formulation;
* the relative-position property that defines rotary embeddings:
  <R(p) q, R(s) k> depends on p − s only; and the norm of every pair is kept;
* the slicing rules of "04 · Megatron-LM 实现" section 5: rotating the full sequence
  and then keeping a rank's rows equals keeping the rows and rotating them at their
  positions — the zigzag chunk pair, the striped split, and, for packed documents,
  positions that restart in every document with the front and mirrored frequency
  slices of each document.
"""
import numpy as np
import pytest

from oracle import partition as P
from oracle import rope as R

COS = {1: 0.5403023058681398, 2: -0.4161468365471424, 3: -0.9899924966004454}
SIN = {1: 0.8414709848078965, 2: 0.9092974268256817, 3: 0.1411200080598672}


@pytest.mark.parametrize("interleaved", [False, True])
def test_hand_computed_rotations(interleaved):
    # d = 4, base 100: θ = (1, 1/10); positions 0..7; pair 0 is (0, 2) or (0, 1)
    d, base = 4, 100.0
    a, b = (0, 1) if interleaved else (0, 2)
    x = np.zeros((8, 1, d))
    x[:, 0, a] = 1.0
    out = R.apply_rope(x, np.arange(8), base, interleaved)
    for p in (1, 2, 3):
        assert abs(out[p, 0, a] - COS[p]) < 1e-15 and abs(out[p, 0, b] - SIN[p]) < 1e-15
    assert np.array_equal(out[0], x[0])          # position 0 leaves the row unchanged
    # the other component of the pair: (0, 1) -> (-sin, cos)
    y = np.zeros((8, 1, d))
    y[:, 0, b] = 1.0
    out = R.apply_rope(y, np.arange(8), base, interleaved)
    for p in (1, 2, 3):
        assert abs(out[p, 0, a] + SIN[p]) < 1e-15 and abs(out[p, 0, b] - COS[p]) < 1e-15
    # the second pair turns ten times slower: position 10 turns it by 1 radian
    z = np.zeros((11, 1, d))
    z[:, 0, 2 if interleaved else 1] = 1.0
    out = R.apply_rope(z, np.arange(11), base, interleaved)
    c1, s1 = (2, 3) if interleaved else (1, 3)
    assert abs(out[10, 0, c1] - COS[1]) < 1e-15 and abs(out[10, 0, s1] - SIN[1]) < 1e-15


@pytest.mark.parametrize("interleaved", [False, True])
def test_complex_form_and_norms(interleaved):
    rng = np.random.default_rng(3)
    t, h, d = 50, 3, 16
    x = rng.standard_normal((t, h, d))
    pos = rng.integers(0, 200000, t)
    out = R.apply_rope(x, pos, 10000.0, interleaved)
    if interleaved:
        z, zo = x[..., 0::2] + 1j * x[..., 1::2], out[..., 0::2] + 1j * out[..., 1::2]
    else:
        z, zo = x[..., : d // 2] + 1j * x[..., d // 2:], out[..., : d // 2] + 1j * out[..., d // 2:]
    theta = pos[:, None, None] * 10000.0 ** (-np.arange(0, d, 2)[None, None, :] / d)
    assert np.max(np.abs(zo - z * np.exp(1j * theta))) < 1e-9
    assert np.max(np.abs(np.abs(zo) - np.abs(z))) < 1e-12


def test_relative_position_property():
    rng = np.random.default_rng(4)
    d = 32
    q, k = rng.standard_normal((1, 1, d)), rng.standard_normal((1, 1, d))
    dots = []
    for p, s in [(10, 3), (107, 100), (7007, 7000), (131071, 131064)]:
        dots.append(float(np.sum(R.apply_rope(q, [p]) * R.apply_rope(k, [s]))))
    assert max(dots) - min(dots) < 1e-9
    other = float(np.sum(R.apply_rope(q, [10]) * R.apply_rope(k, [4])))
    assert abs(other - dots[0]) > 1e-3


def test_zigzag_and_striped_rows_rotate_at_their_global_positions():
    rng = np.random.default_rng(5)
    seq, h, d = 64, 2, 8
    x = rng.standard_normal((seq, h, d))
    full = R.apply_rope(x, np.arange(seq))
    for cp in (2, 4):
        for r in range(cp):
            for rows in (P.zigzag_indices(seq, cp, r), P.striped_indices(seq, cp, r)):
                assert np.array_equal(R.apply_rope(x[rows], rows), full[rows])
    # rotating at local (storage) positions instead is the classic silent bug
    rows = P.zigzag_indices(seq, 4, 1)
    assert np.max(np.abs(R.apply_rope(x[rows], np.arange(len(rows))) - full[rows])) > 0.1


def test_packed_rows_rotate_at_positions_inside_their_document():
    rng = np.random.default_rng(6)
    cu = [0, 16, 48, 56, 64]
    h, d, cp = 2, 8, 2
    x = rng.standard_normal((cu[-1], h, d))
    # each document rotated on its own, positions from 0
    per_doc = np.concatenate([R.apply_rope(x[a:b], np.arange(b - a)) for a, b in zip(cu[:-1], cu[1:])])
    for r in range(cp):
        rows = P.thd_indices(cu, cp, r)
        pos = R.thd_positions(cu, rows)
        assert np.array_equal(R.apply_rope(x[rows], pos), per_doc[rows])
        # the page's description: per document, the front slice of the frequency table
        # [r seg, (r+1) seg) and the mirrored slice [L-(r+1) seg, L-r seg), concatenated
        freqs = []
        for a, b in zip(cu[:-1], cu[1:]):
            L = b - a
            seg = L // (2 * cp)
            table = R.angles(np.arange(L), d)
            freqs.append(np.concatenate([table[r * seg:(r + 1) * seg], table[L - (r + 1) * seg:L - r * seg]]))
        assert np.array_equal(np.concatenate(freqs), R.angles(pos, d))
