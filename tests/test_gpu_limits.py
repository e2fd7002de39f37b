"""Shapes beyond one launch's tables: more than 32 KV segments (streamed in groups of
32 whose partial states are merged; the backward's passes run per group), a 1M-token
share of 131072 local rows (cp = 8), the per-rank size of the pages' 1M-context runs
on 8 devices ("推理系统基础设施（二）…", sections 4-5), and a split launch with more
query tiles than one wave scans at once."""
import numpy as np
import pytest
import torch

import context_causal_attention_zigzag_amd as C
from context_causal_attention_zigzag_amd.rank_share import build_rank_share
import oracle
from oracle import attention as OA
import workloads
from gpu_common import DEV, TOL_BF16, TOL_F32, TOL_LSE_BF16, assert_close, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("n_segs,dtype", [(70, "bf16"), (33, "bf16"), (40, "f32")])
def test_many_segments_stream_and_backward(n_segs, dtype):
    seq, hq, hkv = 2048, 2, 1
    d = 64 if dtype == "f32" else 128
    q = workloads.randn((seq, hq, d), 15, dtype, 0)
    k = workloads.randn((seq, hkv, d), 15, dtype, 1)
    v = workloads.randn((seq, hkv, d), 15, dtype, 2)
    rng = np.random.default_rng(n_segs)
    cuts = np.sort(rng.choice(np.arange(1, seq), n_segs - 1, replace=False))
    bounds = np.concatenate([[0], cuts, [seq]])
    order = rng.permutation(n_segs)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    pos = torch.arange(seq, dtype=torch.int32, device=DEV)
    segs = [C.kv_seg(gk[bounds[i]:bounds[i + 1]], gv[bounds[i]:bounds[i + 1]], pos[bounds[i]:bounds[i + 1]])
            for i in order]
    desc = C.attn_desc(hq, hkv, d, torch.float32 if dtype == "f32" else torch.bfloat16)
    qb = C.q_block(gq, pos)
    o = torch.empty_like(gq)
    lse = torch.empty((seq, hq), dtype=torch.float32, device=DEV)
    say(f"{n_segs} segments stream ({dtype})")
    C.cpattn_stream_fwd(desc, qb, segs, o, lse)           # auto workspace: one partial per group
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_fwd(q, k, v)
    tol_o, tol_l = (TOL_F32, TOL_F32) if dtype == "f32" else (TOL_BF16, TOL_LSE_BF16)
    assert_close(o, o_ref, tol_o, f"{n_segs}-seg O")
    assert_close(lse, l_ref, tol_l, f"{n_segs}-seg LSE")
    if dtype == "f32":
        return
    g = workloads.randn((seq, hq, d), 15, "bf16", 3).to(DEV)
    dq = torch.empty((seq, hq, d), dtype=torch.float32, device=DEV)
    dk = [torch.empty((bounds[i + 1] - bounds[i], hkv, d), dtype=torch.float32, device=DEV) for i in order]
    dv = [torch.empty_like(x) for x in dk]
    ws = torch.empty(max(256, C.cpattn_bwd_workspace_bytes(desc, qb, segs)), dtype=torch.uint8, device=DEV)
    say(f"{n_segs} segments backward")
    C.cpattn_bwd(desc, qb, segs, o, lse, g, dq, dk, dv, ws)
    torch.cuda.synchronize()
    # the first of the dQ launches formed D and left it at the start of the workspace:
    # the delta pass's values bit for bit
    delta_ref = torch.empty((seq, hq), dtype=torch.float32, device=DEV)
    C.cpattn_bwd_delta(desc, o, g, delta_ref)
    torch.cuda.synchronize()
    assert torch.equal(ws[:seq * hq * 4].view(torch.float32).view(seq, hq), delta_ref)
    dq_r, dk_r, dv_r = OA.attention_bwd(q, k, v, g.cpu())
    assert_close(dq, dq_r, TOL_BF16, f"{n_segs}-seg dQ")
    dk_all = torch.empty((seq, hkv, d), dtype=torch.float32)
    dv_all = torch.empty_like(dk_all)
    for j, i in enumerate(order):
        dk_all[bounds[i]:bounds[i + 1]] = dk[j].cpu()
        dv_all[bounds[i]:bounds[i + 1]] = dv[j].cpu()
    assert_close(dk_all, dk_r, TOL_BF16, f"{n_segs}-seg dK")
    assert_close(dv_all, dv_r, TOL_BF16, f"{n_segs}-seg dV")


def test_one_million_token_share_of_131072_rows():
    seq, cp, rank, hq, hkv, d = 1 << 20, 8, 0, 1, 1, 64
    say("1M-token share: inputs")
    q = workloads.randn((seq, hq, d), 16, "bf16", 0)
    k = workloads.randn((seq, hkv, d), 16, "bf16", 1)
    v = workloads.randn((seq, hkv, d), 16, "bf16", 2)
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), cp, rank)
    n = rs.q.shape[0]
    assert n == 131072
    rows = oracle.zigzag_indices(seq, cp, rank)
    assert np.array_equal(rs.q_idx.cpu().numpy(), rows)
    g = workloads.randn((n, hq, d), 16, "bf16", 3)
    say("1M-token share: stream forward + backward (owner segments)")
    o, lse = rs.stream_fwd("owner")
    dq, dk, dv = rs.bwd(o, lse, g.to(DEV))
    torch.cuda.synchronize()
    keys = np.arange(seq)
    local = np.array([0, 1, 4095, 65535, 65536, 65537, 98304, n - 65, n - 2, n - 1])
    say(f"1M-token share: oracle on {len(local)} rows")
    o_r, l_r = OA.attention_fwd(q[torch.as_tensor(rows[local])], k, v, rows[local], keys)
    li = torch.as_tensor(local, device=DEV)
    assert_close(o[li], o_r, TOL_BF16, "1M share O (sampled rows)")
    assert_close(lse[li], l_r, TOL_LSE_BF16, "1M share LSE (sampled rows)")
    dq_r, _, _ = OA.attention_bwd(q[torch.as_tensor(rows[local])], k, v, g[torch.as_tensor(local)], rows[local], keys)
    assert_close(dq[li], dq_r, TOL_BF16, "1M share dQ (sampled rows)")
    # the last 64 keys of the sequence (the end of the rank's own back chunk, owner 0,
    # the first segment in ring order) are seen only by the rank's last 64 rows: their
    # dK / dV follow from those rows alone
    tail = np.arange(n - 64, n)
    say("1M-token share: oracle dK/dV of the last 64 keys")
    dk_r, dv_r = OA.attention_bwd_keys(q[torch.as_tensor(rows[tail])], k, v, g[torch.as_tensor(tail)],
                                       np.arange(seq - 64, seq), rows[tail], keys)
    assert np.array_equal(rs.owners[0].idx[-64:].cpu().numpy(), np.arange(seq - 64, seq))
    assert_close(dk[0][-64:], dk_r, TOL_BF16, "1M share dK (last 64 keys)")
    assert_close(dv[0][-64:], dv_r, TOL_BF16, "1M share dV (last 64 keys)")
    # every key: the dV rows sum to the summed upstream gradient (probabilities sum to 1)
    dv_sum = sum(x.double().sum(0) for x in dv).cpu()
    g_sum = g.double().sum(0)
    tol = 3 * 2.0 ** -9 * g.double().pow(2).sum(0).sqrt()
    say(f"1M share: sum dV vs sum G max err {float((dv_sum - g_sum).abs().max()):.3e}")
    assert float(((dv_sum - g_sum).abs() - tol).max()) <= 0.0


def test_split_numbering_beyond_one_wave():
    # S = 16384 on one rank (cp = 1), two heads: four-wave work-groups of 128 rows, 128
    # query tiles whose 256 KV tiles are split (256 query work-groups for 512 slots), so
    # the dense split numbering scans its counts in two chunks of one wave.  Forward and
    # dQ on sampled rows against the oracle.
    seq, cp, hq, d = 16384, 1, 2, 64
    q = workloads.randn((seq, hq, d), 23, "bf16", 0)
    k = workloads.randn((seq, hq, d), 23, "bf16", 1)
    v = workloads.randn((seq, hq, d), 23, "bf16", 2)
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), cp, 0)
    ws = rs.stream_workspace("owner")
    assert ws is not None, "expected a split launch"
    say("split numbering over 128 query tiles: stream")
    o, lse = rs.stream_fwd("owner", workspace=ws)
    g = workloads.randn((seq // cp, hq, d), 23, "bf16", 3).to(DEV)
    desc = rs.desc()
    qblk = C.q_block(rs.q, rs.q_idx, rs.q_doc)
    segs = [s for s, _, _ in rs.segments("owner")]
    delta = torch.empty((seq // cp, hq), dtype=torch.float32, device=DEV)
    C.cpattn_bwd_delta(desc, o, g, delta)
    n_ws = C.cpattn_bwd_dq_workspace_bytes(desc, qblk, segs)
    assert n_ws > 0, "expected a split dQ pass"
    dq = torch.empty((seq // cp, hq, d), dtype=torch.float32, device=DEV)
    say("split numbering over 128 query tiles: dQ")
    C.cpattn_bwd_dq(desc, qblk, segs, lse, delta, g, dq, torch.empty(n_ws, dtype=torch.uint8, device=DEV))
    # the dQ pass that forms D itself: the same D and dQ bit for bit (d = 64, split)
    delta2 = torch.full_like(delta, float("nan"))
    dq2 = torch.empty_like(dq)
    C.cpattn_bwd_dq_delta(desc, qblk, segs, o, lse, g, delta2, dq2, torch.empty(n_ws, dtype=torch.uint8, device=DEV))
    torch.cuda.synchronize()
    assert torch.equal(delta2, delta) and torch.equal(dq2, dq)
    local = rs.q_idx.cpu().numpy().astype(np.int64)
    pick = np.unique(np.linspace(0, len(local) - 1, 40).astype(np.int64))
    rows = local[pick]
    keys = np.arange(seq)
    o_ref, l_ref = OA.attention_fwd(q[torch.as_tensor(rows)], k, v, rows, keys)
    sel = torch.as_tensor(pick, device=DEV)
    assert_close(o[sel], o_ref, TOL_BF16, "128-tile split O")
    assert_close(lse[sel], l_ref, TOL_LSE_BF16, "128-tile split LSE")
    # dQ of those rows, with D formed from the bf16 O the GPU saved
    g_rows = g[sel].cpu()
    dq_ref, _, _ = OA.attention_bwd(q[torch.as_tensor(rows)], k, v, g_rows, rows, keys, o_saved=o[sel].cpu())
    assert_close(dq[sel], dq_ref, TOL_BF16, "128-tile split dQ")
