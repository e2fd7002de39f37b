"""Full-size workloads in the launch configuration the benchmark times, checked on
sampled rows against the oracle (which evaluates those rows against every key), and
the two forward forms checked against each other on every row.  The 128K and packed
backward passes are checked on sampled query rows (dQ) and, for dK / dV, through two
identities of the softmax Jacobian that hold at any size (per document when packed)."""
import numpy as np
import pytest
import torch

from context_causal_attention_zigzag_amd.rank_share import build_rank_share
import oracle
import workloads
from gpu_common import (DEV, TOL_BF16, TOL_LSE_BF16, assert_close, oracle_fwd_rows, say)
from oracle import attention as OA

pytestmark = pytest.mark.gpu


def sample_local_rows(n, extra, seed):
    base = [0, 1, 31, 32, 63, 64, 127, 128, n // 2 - 1, n // 2, n // 2 + 1, n - 2, n - 1]
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([base, rng.integers(0, n, extra)]))


def test_s128k_rank0_sampled():
    w = workloads.WORKLOADS["s128k"]
    say("s128k: generating inputs")
    q, k, v = workloads.full_qkv(w)
    say("s128k: partition + stream")
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), w.cp, 0)
    o, lse = rs.stream_fwd("chunk")
    torch.cuda.synchronize()
    say("s128k: tile + merge")
    edges, parts = rs.alloc_tile_buffers("chunk")
    assert len(edges) == 2 * w.cp + 1
    rs.tile_fwd(edges, parts)
    o2, l2 = rs.merge(edges, parts)
    torch.cuda.synchronize()
    del parts
    local = sample_local_rows(rs.q.shape[0], 19, 3)
    rows = rs.q_idx.cpu().numpy()[local]
    assert np.array_equal(rows, oracle.zigzag_indices(w.seq, w.cp, 0)[local])
    say(f"s128k: oracle on {len(local)} rows")
    o_ref, l_ref = oracle_fwd_rows(q, k, v, rows)
    li = torch.as_tensor(local, device=DEV)
    assert_close(o[li], o_ref, TOL_BF16, "s128k stream O (sampled)")
    assert_close(lse[li], l_ref, TOL_LSE_BF16, "s128k stream LSE (sampled)")
    assert_close(o2[li], o_ref, TOL_BF16, "s128k tile O (sampled)")
    assert_close(l2[li], l_ref, TOL_LSE_BF16, "s128k tile LSE (sampled)")
    # every row: the two forward forms agree
    assert_close(o2, o.float(), TOL_BF16, "s128k tile vs stream O (all rows)")
    assert_close(l2, lse, TOL_LSE_BF16, "s128k tile vs stream LSE (all rows)")


def test_thd64k_rank1_sampled():
    w = workloads.WORKLOADS["thd64k"]
    cu = workloads.cu_seqlens_from_lengths(workloads.thd_lengths(w.seed))
    q, k, v = workloads.full_qkv(w)
    say("thd64k: partition + stream")
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), w.cp, 1, cu)
    o, lse = rs.stream_fwd("owner")
    edges, parts = rs.alloc_tile_buffers("owner")
    rs.tile_fwd(edges, parts)
    o2, l2 = rs.merge(edges, parts)
    torch.cuda.synchronize()
    rows_all = oracle.thd_indices(cu, w.cp, 1)
    assert np.array_equal(rs.q_idx.cpu().numpy(), rows_all)
    assert np.array_equal(rs.q_doc.cpu().numpy(), oracle.thd_doc_ids(cu, rows_all))
    # sampled rows: both ends of every document's two slices plus random rows
    docs = oracle.thd_doc_ids(cu, rows_all)
    ends = np.flatnonzero(np.diff(docs)) 
    local = np.unique(np.concatenate([sample_local_rows(len(rows_all), 16, 4), ends, ends + 1]))
    rows = rows_all[local]
    say(f"thd64k: oracle on {len(local)} rows")
    all_docs = oracle.thd_doc_ids(cu, np.arange(w.seq))
    o_ref, l_ref = oracle_fwd_rows(q, k, v, rows, cu, all_docs)
    li = torch.as_tensor(local, device=DEV)
    assert_close(o[li], o_ref, TOL_BF16, "thd64k stream O (sampled)")
    assert_close(lse[li], l_ref, TOL_LSE_BF16, "thd64k stream LSE (sampled)")
    assert_close(o2[li], o_ref, TOL_BF16, "thd64k tile O (sampled)")
    assert_close(o2, o.float(), TOL_BF16, "thd64k tile vs stream O (all rows)")
    assert_close(l2, lse, TOL_LSE_BF16, "thd64k tile vs stream LSE (all rows)")


def test_s128k_rank0_bwd_sampled():
    w = workloads.WORKLOADS["s128k"]
    say("s128k bwd: generating inputs")
    q, k, v = workloads.full_qkv(w)
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), w.cp, 0)
    n = rs.q.shape[0]
    g = workloads.randn((n, w.hq, w.d), w.seed, "bf16", 3)
    say("s128k bwd: stream forward + backward (chunk segments, as timed)")
    o, lse = rs.stream_fwd("chunk")
    dq, dk, dv = rs.bwd(o, lse, g.to(DEV), granularity="chunk")
    torch.cuda.synchronize()
    # dQ of sampled rows: the oracle runs those rows' own forward and backward over
    # every key
    local = sample_local_rows(n, 13, 5)
    rows = rs.q_idx.cpu().numpy()[local]
    say(f"s128k bwd: oracle dQ on {len(local)} rows")
    dq_r, _, _ = OA.attention_bwd(q[torch.as_tensor(rows)], k, v, g[torch.as_tensor(local)], rows,
                                  np.arange(w.seq))
    assert_close(dq[torch.as_tensor(local, device=DEV)], dq_r, TOL_BF16, "s128k dQ (sampled)")
    # Every visible row's probabilities sum to 1, so the dV rows of all keys of a kv
    # head sum to the upstream gradient summed over the local rows and the head's query
    # group.  The kernels round P to bf16 (relative error <= 2^-9 per probability, of
    # either sign), which moves a row's sum by at most 2^-9; over the rows these errors
    # add like a random walk, so each element may differ by 3 * 2^-9 * sqrt(sum G^2).
    grp = w.hq // w.hkv
    g64 = g.double().reshape(n, w.hkv, grp, w.d)
    g_sum = g64.sum((0, 2))
    dv_tol = 3 * 2.0 ** -9 * g64.pow(2).sum((0, 2)).sqrt()
    dv_sum = sum(x.double().sum(0) for x in dv).cpu()
    dv_excess = float(((dv_sum - g_sum).abs() - dv_tol).max())
    # Every row of dS sums to 0 except for D, which uses O rounded to bf16: per row
    # G.(O - bf16(O)) is at most 2^-9 |G||O|; times the scale and the row's q, summed
    # over the rows like a random walk, that is far below 0.5 (the sums of wrong dK
    # rows are of the order of sqrt(rows) = 256).
    dk_sum = sum(x.double().sum(0) for x in dk).cpu()
    dk_max = float(dk_sum.abs().max())
    say(f"s128k bwd: sum dV vs sum G max err {float((dv_sum - g_sum).abs().max()):.3e} "
        f"(tolerance >= {float(dv_tol.min()):.3f}); |sum dK| max {dk_max:.3e}")
    assert dv_excess <= 0.0, dv_excess
    assert dk_max <= 0.5, dk_max


def test_thd64k_rank1_bwd_sampled():
    w = workloads.WORKLOADS["thd64k"]
    cu = workloads.cu_seqlens_from_lengths(workloads.thd_lengths(w.seed))
    say("thd64k bwd: generating inputs")
    q, k, v = workloads.full_qkv(w)
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), w.cp, 1, cu)
    n = rs.q.shape[0]
    g = workloads.randn((n, w.hq, w.d), w.seed, "bf16", 3)
    say("thd64k bwd: stream forward + backward (owner segments, as timed)")
    o, lse = rs.stream_fwd("owner")
    dq, dk, dv = rs.bwd(o, lse, g.to(DEV), granularity="owner")
    torch.cuda.synchronize()
    rows_all = rs.q_idx.cpu().numpy()
    q_docs = rs.q_doc.cpu().numpy()
    all_docs = oracle.thd_doc_ids(cu, np.arange(w.seq))
    # dQ of sampled rows (both ends of every document's slices among them) against the
    # oracle over every key with the document mask
    ends = np.flatnonzero(np.diff(q_docs))
    local = np.unique(np.concatenate([sample_local_rows(n, 13, 6), ends, ends + 1]))
    rows = rows_all[local]
    say(f"thd64k bwd: oracle dQ on {len(local)} rows")
    dq_r, _, _ = OA.attention_bwd(q[torch.as_tensor(rows)], k, v, g[torch.as_tensor(local)], rows,
                                  np.arange(w.seq), q_docs[local], all_docs, mask=OA.MASK_CAUSAL_DOC)
    assert_close(dq[torch.as_tensor(local, device=DEV)], dq_r, TOL_BF16, "thd64k dQ (sampled)")
    # Per document: a row sees keys of its own document only and its probabilities sum
    # to 1, so the dV rows of a document's keys (over all owners) sum to G summed over
    # the local rows of that document, and its dK rows to 0 (the tolerances are those
    # of the 128K test, per document).
    n_docs = len(cu) - 1
    dv_doc = torch.zeros((n_docs, w.hkv, w.d), dtype=torch.float64)
    dk_doc = torch.zeros_like(dv_doc)
    for (seg, (owner, _), (a, b)), dk_s, dv_s in zip(rs.segments("owner"), dk, dv):
        kd = torch.as_tensor(rs.owners[owner].doc[a:b].cpu().numpy(), dtype=torch.long)
        dv_doc.index_add_(0, kd, dv_s.double().cpu())
        dk_doc.index_add_(0, kd, dk_s.double().cpu())
    qd = torch.as_tensor(q_docs, dtype=torch.long)
    g64 = g.double().reshape(n, w.hkv, w.hq // w.hkv, w.d).sum(2)
    g_doc = torch.zeros_like(dv_doc).index_add_(0, qd, g64)
    g2_doc = torch.zeros_like(dv_doc).index_add_(0, qd, g.double().reshape(n, w.hkv, -1, w.d).pow(2).sum(2))
    dv_tol = 3 * 2.0 ** -9 * g2_doc.sqrt()
    dv_excess = float(((dv_doc - g_doc).abs() - dv_tol).max())
    dk_max = float(dk_doc.abs().max())
    say(f"thd64k bwd: per-document sum dV vs sum G max err {float((dv_doc - g_doc).abs().max()):.3e}; "
        f"|sum dK| max {dk_max:.3e}")
    assert dv_excess <= 0.0, dv_excess
    assert dk_max <= 0.5, dk_max
