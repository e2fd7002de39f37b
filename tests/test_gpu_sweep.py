"""Seeded sweep of mixed shapes: each case draws a layout (zigzag, striped or packed
documents), cp, rank, query/KV head grouping, head dim and lengths with ragged tails,
then compares the streaming forward, the tile + merge forward (owner and chunk edges,
with and without KV splits) and, for bf16, dQ and every owner's dK/dV with the
oracle element by element.  The fixed cases elsewhere pin each feature on its own;
this one crosses them (a striped share with grouped heads at d = 64, a packed share
whose documents end inside a tile at cp = 3, ...).  Lengths reach a few thousand
tokens, so the longer cases take the KV-split plans, and every fourth case is planned
for two compute units, which gives the forward and dQ launches eight-wave work-groups.

CPATTN_SWEEP_CASES, CPATTN_SWEEP_SEED and CPATTN_SWEEP_LONG=1 (lengths up to about
1.75x longer, oracle work per case up to 8e7 pairs) widen the sweep; the defaults
keep it to seconds."""
import os

import numpy as np
import pytest
import torch

from context_causal_attention_zigzag_amd.rank_share import build_rank_share, ring_order
import oracle
from oracle import attention as OA
import workloads
from gpu_common import DEV, TOL_BF16, TOL_F32, TOL_LSE_BF16, assert_close, say

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("CPATTN_SWEEP_CASES", "48"))
SEED = int(os.environ.get("CPATTN_SWEEP_SEED", "20261202"))
LONG = os.environ.get("CPATTN_SWEEP_LONG", "0") == "1"
# local rows x keys x query heads: keeps each oracle pass to seconds
MAX_PAIRS = 8e7 if LONG else 3e7


def draw_cases(seed=SEED):
    rng = np.random.default_rng(seed)
    cases = []
    layouts = ("zigzag", "striped", "packed")
    while len(cases) < N_CASES:
        i = len(cases)
        layout = layouts[i % 3]
        cp = int(rng.integers(1, 5))
        hkv = int(rng.choice([1, 2, 4]))
        hq = hkv * int(rng.integers(1, 5))
        d = int(rng.choice([64, 128]))
        dtype = "f32" if i % 6 == 5 else "bf16"
        lengths = None
        if layout == "zigzag":
            seq = 2 * cp * int(rng.integers(3, 1400 if LONG else 800))
        elif layout == "striped":
            seq = cp * int(rng.integers(5, 2600 if LONG else 1500))
        else:
            n_docs = int(rng.integers(1, 9))
            # a zero-length document now and then; otherwise lengths with ragged tails
            lengths = [2 * cp * (0 if rng.random() < 0.1 else int(rng.integers(1, 500 if LONG else 300)))
                       for _ in range(n_docs)]
            seq = sum(lengths)
            if seq == 0:
                continue
        if seq * seq * hq / cp > MAX_PAIRS:
            continue
        rank = int(rng.integers(0, cp))
        cases.append(dict(id=f"{i:02d}-{layout}-s{seq}-cp{cp}r{rank}-h{hq}x{hkv}-d{d}-{dtype}",
                          layout=layout, seq=seq, cp=cp, rank=rank, hq=hq, hkv=hkv, d=d,
                          dtype=dtype, lengths=lengths, seed=100 + i, few_cus=i % 4 == 3))
    return cases


CASES = draw_cases()


def share_rows(c, cu):
    if c["layout"] == "zigzag":
        return lambda r: oracle.zigzag_indices(c["seq"], c["cp"], r)
    if c["layout"] == "striped":
        return lambda r: oracle.striped_indices(c["seq"], c["cp"], r)
    return lambda r: oracle.thd_indices(cu, c["cp"], r)


@pytest.mark.parametrize("c", CASES, ids=[c["id"] for c in CASES])
def test_sweep_case(c, monkeypatch):
    if c["few_cus"]:
        monkeypatch.setenv("CPATTN_NUM_CUS", "2")
    say(f"sweep {c['id']}{' (planned for 2 CUs)' if c['few_cus'] else ''}")
    seq, cp, rank, hq, hkv, d, dt = c["seq"], c["cp"], c["rank"], c["hq"], c["hkv"], c["d"], c["dtype"]
    q = workloads.randn((seq, hq, d), c["seed"], dt, 0)
    k = workloads.randn((seq, hkv, d), c["seed"], dt, 1)
    v = workloads.randn((seq, hkv, d), c["seed"], dt, 2)
    cu = None if c["lengths"] is None else workloads.cu_seqlens_from_lengths(c["lengths"])
    rows_of = share_rows(c, cu)
    rows = rows_of(rank)
    keys = np.arange(seq)
    kw = {}
    if cu is not None:
        kw = dict(q_doc=oracle.thd_doc_ids(cu, rows), k_doc=oracle.thd_doc_ids(cu, keys),
                  mask=OA.MASK_CAUSAL_DOC)
    tq = q[torch.as_tensor(rows)]
    o_ref, l_ref = OA.attention_fwd(tq, k, v, rows, keys, kw.get("q_doc"), kw.get("k_doc"),
                                    kw.get("mask", OA.MASK_CAUSAL))
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), cp, rank, cu,
                          striped=c["layout"] == "striped")
    assert np.array_equal(rs.q_idx.cpu().numpy(), rows)
    tol_o, tol_l = (TOL_F32, TOL_F32) if dt == "f32" else (TOL_BF16, TOL_LSE_BF16)
    for gran in ("owner", "chunk"):
        for ws in ("auto", None):
            tag = f"{c['id']} {gran}/{'split' if ws else 'nosplit'}"
            o, lse = rs.stream_fwd(gran, workspace=ws)
            edges, parts = rs.alloc_tile_buffers(gran)
            rs.tile_fwd(edges, parts, workspace=ws)
            o2, l2 = rs.merge(edges, parts)
            torch.cuda.synchronize()
            assert_close(o, o_ref, tol_o, f"{tag} stream O")
            assert_close(lse, l_ref, tol_l, f"{tag} stream LSE")
            assert_close(o2, o_ref, tol_o, f"{tag} tile O")
            assert_close(l2, l_ref, tol_l, f"{tag} tile LSE")
    if dt != "bf16":
        return   # the backward takes bf16 inputs only
    g = workloads.randn((len(rows), hq, d), c["seed"], dt, 3)
    o, lse = rs.stream_fwd("owner")
    dq, dk, dv = rs.bwd(o, lse, g.to(DEV))
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = OA.attention_bwd(tq, k, v, g, rows, keys, **kw)
    assert_close(dq, dq_r, TOL_BF16, f"{c['id']} dQ")
    for i, owner in enumerate(ring_order(cp, rank)):
        orow = rows_of(owner)
        assert np.array_equal(rs.owners[owner].idx.cpu().numpy(), orow)
        assert_close(dk[i], dk_r[orow], TOL_BF16, f"{c['id']} dK owner {owner}")
        assert_close(dv[i], dv_r[orow], TOL_BF16, f"{c['id']} dV owner {owner}")
