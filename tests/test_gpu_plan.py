"""Ranked launches planned once (the plan kernel) against the same launches ranked by
every work-group, and a packed share with more query tiles than a work-group can rank.

A planned launch runs exactly the work items of the in-kernel ranking (same order,
same tiles per work item, no KV splits), so its outputs must be bit-identical; the
oracle comparisons of the packed tests cover both paths as well.
"""
import numpy as np
import pytest
import torch

import context_causal_attention_zigzag_amd as C
from context_causal_attention_zigzag_amd.rank_share import build_rank_share
import oracle
from oracle import attention as OA
import workloads
from gpu_common import DEV, TOL_BF16, TOL_LSE_BF16, assert_close, say

pytestmark = pytest.mark.gpu

LENGTHS = [8, 64, 136, 0, 16, 256, 8, 32, 520, 1024, 40, 4, 300]


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (16, 8, 64)])
def test_planned_ranking_matches_in_kernel_ranking(monkeypatch, hq, hkv, d):
    # two compute units: the query tiles take many rounds, so a workspace gets a plan
    monkeypatch.setenv("CPATTN_NUM_CUS", "2")
    cu = workloads.cu_seqlens_from_lengths(LENGTHS)
    total = int(cu[-1])
    q = workloads.randn((total, hq, d), 21, "bf16", 0)
    k = workloads.randn((total, hkv, d), 21, "bf16", 1)
    v = workloads.randn((total, hkv, d), 21, "bf16", 2)
    g = workloads.randn((total // 2, hq, d), 21, "bf16", 3).to(DEV)
    for r in range(2):
        rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), 2, r, cu)
        desc = rs.desc()
        qblk = C.q_block(rs.q, rs.q_idx, rs.q_doc)
        segs = [s for s, _, _ in rs.segments("owner")]
        ws_s = rs.stream_workspace("owner")
        assert ws_s is not None, "expected a planned launch"
        say(f"plan hq={hq} d={d} rank={r}: stream")
        o1, l1 = rs.stream_fwd("owner", workspace=ws_s)
        o0, l0 = rs.stream_fwd("owner", workspace=None)
        torch.cuda.synchronize()
        assert torch.equal(o1, o0) and torch.equal(l1, l0)
        say(f"plan hq={hq} d={d} rank={r}: tile")
        edges, parts1 = rs.alloc_tile_buffers("owner")
        _, parts0 = rs.alloc_tile_buffers("owner")
        rs.tile_fwd(edges, parts1, workspace=rs.tile_workspace(edges))
        rs.tile_fwd(edges, parts0, workspace=None)
        torch.cuda.synchronize()
        for (a1, b1), (a0, b0) in zip(parts1, parts0):
            assert torch.equal(a1, a0) and torch.equal(b1, b0)
        say(f"plan hq={hq} d={d} rank={r}: dQ")
        delta = torch.empty((rs.q.shape[0], hq), dtype=torch.float32, device=DEV)
        C.cpattn_bwd_delta(desc, o1, g, delta)
        n_ws = C.cpattn_bwd_dq_workspace_bytes(desc, qblk, segs)
        assert n_ws > 0
        ws_q = torch.empty(n_ws, dtype=torch.uint8, device=DEV)
        dq1 = torch.empty((rs.q.shape[0], hq, d), dtype=torch.float32, device=DEV)
        dq0 = torch.empty_like(dq1)
        C.cpattn_bwd_dq(desc, qblk, segs, l1, delta, g, dq1, ws_q)
        C.cpattn_bwd_dq(desc, qblk, segs, l1, delta, g, dq0, None)
        torch.cuda.synchronize()
        assert torch.equal(dq1, dq0)


def test_more_query_tiles_than_a_work_group_ranks():
    # 1M tokens in 64 documents of 16384, cp = 2: 524288 local rows, 2048 query tiles of
    # 256 rows; only a planned launch orders them by work (the in-kernel ranking stops at
    # 1024).  Forward rows sampled against the oracle; planned and unplanned bit-equal.
    cp, hq, d = 2, 8, 64
    lengths = [16384] * 64
    cu = workloads.cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    q = workloads.randn((total, hq, d), 22, "bf16", 0)
    k = workloads.randn((total, hq, d), 22, "bf16", 1)
    v = workloads.randn((total, hq, d), 22, "bf16", 2)
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), cp, 0, cu)
    ws = rs.stream_workspace("owner")
    assert ws is not None, "expected a planned launch"
    say("plan 2048 query tiles: stream planned / unplanned")
    o1, l1 = rs.stream_fwd("owner", workspace=ws)
    o0, l0 = rs.stream_fwd("owner", workspace=None)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)
    # 12 rows in each of four documents, against those documents' keys only (a row sees
    # nothing outside its document, so the restriction is exact)
    local = rs.q_idx.cpu().numpy().astype(np.int64)
    ldoc = oracle.thd_doc_ids(cu, local)
    pick = np.concatenate([np.flatnonzero(ldoc == dd)[np.linspace(0, 8191, 12).astype(np.int64)]
                           for dd in (0, 21, 42, 63)])
    rows = local[pick]
    keys = np.concatenate([np.arange(cu[dd], cu[dd + 1]) for dd in (0, 21, 42, 63)])
    kt = torch.as_tensor(keys)
    o_ref, l_ref = OA.attention_fwd(q[torch.as_tensor(rows)], k[kt], v[kt], rows, keys,
                                    oracle.thd_doc_ids(cu, rows), oracle.thd_doc_ids(cu, keys),
                                    OA.MASK_CAUSAL_DOC)
    sel = torch.as_tensor(pick, device=DEV)
    assert_close(o1[sel], o_ref, TOL_BF16, "2048 tiles O")
    assert_close(l1[sel], l_ref, TOL_LSE_BF16, "2048 tiles LSE")
