"""Pins for the partition oracle (CPU only).

What fixes the answer: the cp=2 chunk assignment printed on the "Context
Parallelism (CP)" page (section 4), the permutation and one-light/one-heavy
properties the zigzag is introduced for, the closed-form visible-pair count
S(S+1)/(2cp) that makes every rank's causal work equal, and a second formulation of
the per-document split (reshape each document into 2cp chunks and pick r, 2cp-1-r).
"""
import json
import os

import numpy as np
import pytest

from oracle import partition as P
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_zigzag_cp2_matches_printed_assignment():
    g = json.load(open(os.path.join(GOLDEN, "zigzag_cp2.json")))
    seq = 512
    chunk = seq // (2 * g["cp"])
    for r, chunks in g["rank_chunks"].items():
        want = np.concatenate([np.arange(c * chunk, (c + 1) * chunk) for c in chunks])
        got = P.zigzag_indices(seq, g["cp"], int(r))
        assert np.array_equal(got, want)


@pytest.mark.parametrize("seq,cp", [(512, 2), (8192, 4), (64, 8), (48, 3), (8, 1)])
def test_zigzag_union_is_permutation(seq, cp):
    rows = np.concatenate([P.zigzag_indices(seq, cp, r) for r in range(cp)])
    assert np.array_equal(np.sort(rows), np.arange(seq))


@pytest.mark.parametrize("seq,cp", [(512, 2), (8192, 4), (131072, 8)])
def test_zigzag_light_and_heavy_chunk(seq, cp):
    chunk = seq // (2 * cp)
    for r in range(cp):
        rows = P.zigzag_indices(seq, cp, r)
        first, second = rows[:chunk] // chunk, rows[chunk:] // chunk
        assert np.all(first == first[0]) and np.all(second == second[0])
        assert first[0] < cp <= second[0]
        assert first[0] + second[0] == 2 * cp - 1


@pytest.mark.parametrize("seq,cp,pairs", [(512, 2, 65664), (8192, 4, 8389632), (131072, 8, 1073750016)])
def test_zigzag_equal_causal_work(seq, cp, pairs):
    # query at global position p sees keys 0..p of the whole sequence
    for r in range(cp):
        rows = P.zigzag_indices(seq, cp, r)
        assert int(np.sum(rows + 1)) == pairs == seq * (seq + 1) // (2 * cp)


def test_zigzag_nonempty_chunk_edges():
    # chunk-level edges (Q chunk, KV chunk) with at least one visible pair: 2cp+1 per rank
    for seq, cp in [(512, 2), (8192, 4), (131072, 8)]:
        for r in range(cp):
            qc = [r, 2 * cp - 1 - r]
            edges = sum(1 for a in qc for b in range(2 * cp) if b <= a)
            assert edges == 2 * cp + 1


def test_zigzag_alignment_errors():
    with pytest.raises(ValueError):
        P.zigzag_indices(100, 4, 0)
    with pytest.raises(ValueError):
        P.zigzag_indices(64, 4, 4)


def _thd_by_reshape(cu, cp, r):
    out = []
    for a, b in zip(cu[:-1], cu[1:]):
        doc = np.arange(a, b).reshape(2 * cp, -1)
        out.append(doc[[r, 2 * cp - 1 - r]].ravel())
    return np.concatenate(out) if out else np.zeros(0, np.int64)


@pytest.mark.parametrize("seed", [0, 1, 4])
def test_thd_matches_per_document_zigzag(seed):
    cu = workloads.cu_seqlens_from_lengths(workloads.thd_lengths(seed))
    for r in range(4):
        assert np.array_equal(P.thd_indices(cu, 4, r), _thd_by_reshape(cu, 4, r))


def test_thd_single_document_is_zigzag():
    for seq, cp in [(512, 2), (8192, 4)]:
        for r in range(cp):
            assert np.array_equal(P.thd_indices([0, seq], cp, r), P.zigzag_indices(seq, cp, r))


def test_thd_cp1_is_identity():
    cu = workloads.cu_seqlens_from_lengths([8, 16, 24])
    assert np.array_equal(P.thd_indices(cu, 1, 0), np.arange(48))


def test_thd_union_pairs_and_docs():
    cu = workloads.cu_seqlens_from_lengths(workloads.thd_lengths(4))
    lengths = np.diff(cu).astype(np.int64)
    cp = 4
    want_pairs = int(np.sum(lengths * (lengths + 1))) // (2 * cp)
    allrows = []
    for r in range(cp):
        rows = P.thd_indices(cu, cp, r)
        allrows.append(rows)
        docs = P.thd_doc_ids(cu, rows)
        assert np.array_equal(docs, np.searchsorted(cu, rows, side="right") - 1)
        assert np.all(np.diff(rows) > 0)          # ascending within the rank
        offs = rows - cu[docs]
        assert int(np.sum(offs + 1)) == want_pairs  # equal packed causal work
    assert np.array_equal(np.sort(np.concatenate(allrows)), np.arange(cu[-1]))


def test_thd_rope_slice_description():
    # front slice [r*seg, (r+1)*seg) ++ mirrored slice [L-(r+1)*seg, L-r*seg) of each document
    cu = [0, 16, 48, 56]
    cp, r = 2, 1
    want = [4, 5, 6, 7, 8, 9, 10, 11,
            16 + 8, 16 + 9, 16 + 10, 16 + 11, 16 + 12, 16 + 13, 16 + 14, 16 + 15,
            16 + 16, 16 + 17, 16 + 18, 16 + 19, 16 + 20, 16 + 21, 16 + 22, 16 + 23,
            48 + 2, 48 + 3, 48 + 4, 48 + 5]
    assert P.thd_indices(cu, cp, r).tolist() == want


def test_thd_alignment_errors():
    with pytest.raises(ValueError):
        P.thd_indices([0, 12], 4, 0)
    with pytest.raises(ValueError):
        P.thd_indices([0, 16, 8], 2, 0)


# ---------------------------------------------------------------- striped split
def test_striped_matches_printed_interleave():
    g = json.load(open(os.path.join(GOLDEN, "striped_cp4.json")))
    for r, prefix in g["printed_prefixes"].items():
        got = P.striped_indices(64, g["cp"], int(r))
        assert got[: len(prefix)].tolist() == prefix


@pytest.mark.parametrize("seq,cp", [(64, 4), (8192, 4), (48, 3), (8, 1), (24, 8)])
def test_striped_union_is_permutation_and_ascending(seq, cp):
    parts = [P.striped_indices(seq, cp, r) for r in range(cp)]
    assert all(np.all(np.diff(p) > 0) for p in parts)
    assert all(len(p) == seq // cp for p in parts)
    assert np.array_equal(np.sort(np.concatenate(parts)), np.arange(seq))


@pytest.mark.parametrize("seq,cp", [(64, 4), (96, 3), (8192, 4)])
def test_striped_pair_counts(seq, cp):
    # rank r holds positions r + cp t, t < n = seq / cp; each sees its prefix of keys:
    # n (r + 1) + cp n (n - 1) / 2 visible pairs, so rank r + 1 carries n more pairs
    # than rank r (nearly balanced, unlike the exact balance of the zigzag split)
    n = seq // cp
    from oracle import attention as A
    counts = []
    for r in range(cp):
        rows = P.striped_indices(seq, cp, r)
        want = n * (r + 1) + cp * n * (n - 1) // 2
        if seq <= 128:
            assert int(A.visible_mask(rows, np.arange(seq)).sum()) == want
        assert int(np.sum(rows + 1)) == want
        counts.append(want)
    assert counts[-1] - counts[0] == (cp - 1) * n


def test_striped_alignment_errors():
    with pytest.raises(ValueError):
        P.striped_indices(10, 4, 0)
    with pytest.raises(ValueError):
        P.striped_indices(16, 4, 4)
