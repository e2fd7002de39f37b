"""Backward parity: dQ and the per-owner dK/dV sums vs the oracle's float64 gradients."""
import numpy as np
import pytest
import torch

from context_causal_attention_zigzag_amd.rank_share import build_rank_share, ring_order
import oracle
from oracle import attention as OA
import workloads
from gpu_common import DEV, TOL_BF16, assert_close, rank_rows, say

pytestmark = pytest.mark.gpu


def run_bwd(q, k, v, g_full, cp, rank, cu=None):
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), cp, rank, cu)
    rows, qdoc = rank_rows(q.shape[0], cp, rank, cu)
    g = g_full[torch.as_tensor(rows)]
    o, lse = rs.stream_fwd("owner")
    dq, dk, dv = rs.bwd(o, lse, g.to(DEV))
    torch.cuda.synchronize()
    return rs, rows, g, dq, dk, dv


def check_bwd(name, q, k, v, g_full, cp, rank, cu=None):
    say(f"{name} bwd rank={rank}")
    rs, rows, g, dq, dk, dv = run_bwd(q, k, v, g_full, cp, rank, cu)
    seq = q.shape[0]
    kw = {}
    if cu is not None:
        kw = dict(q_doc=oracle.thd_doc_ids(cu, rows), k_doc=oracle.thd_doc_ids(cu, np.arange(seq)),
                  mask=OA.MASK_CAUSAL_DOC)
    dq_r, dk_r, dv_r = OA.attention_bwd(q[torch.as_tensor(rows)], k, v, g, rows, np.arange(seq), **kw)
    assert_close(dq, dq_r, TOL_BF16, f"{name} r{rank} dQ")
    for (o_idx, owner) in enumerate(ring_order(cp, rank)):
        orow = rs.owners[owner].idx.cpu().numpy()
        assert_close(dk[o_idx], dk_r[orow], TOL_BF16, f"{name} r{rank} dK owner {owner}")
        assert_close(dv[o_idx], dv_r[orow], TOL_BF16, f"{name} r{rank} dV owner {owner}")
    return rs, dk, dv


@pytest.fixture(scope="module")
def bwd8k():
    w = workloads.WORKLOADS["bwd8k"]
    q, k, v = workloads.full_qkv(w)
    g = workloads.randn((w.seq, w.hq, w.d), w.grad_seed, w.dtype, 3)
    return w, q, k, v, g


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_bwd8k_rank(bwd8k, rank):
    w, q, k, v, g = bwd8k
    check_bwd("bwd8k", q, k, v, g, w.cp, rank)


def test_bwd8k_unsplit_dq_pass(bwd8k):
    # a workspace holding only rowsum(dO*O) runs the dQ pass without KV splits
    w, q, k, v, g = bwd8k
    import context_causal_attention_zigzag_amd as C
    rs, rows, gr, dq_split, dk_s, dv_s = run_bwd(q, k, v, g, w.cp, 1)
    o, lse = rs.stream_fwd("owner")
    dq, dk, dv, _ = rs.alloc_bwd_buffers()
    small = torch.empty(rs.q.shape[0] * w.hq * 4, dtype=torch.uint8, device=DEV)
    say("bwd8k unsplit dQ pass")
    segs = [s_ for s_, _, _ in rs.segments("owner")]
    C.cpattn_bwd(rs.desc(), C.q_block(rs.q, rs.q_idx), segs, o, lse, gr.to(DEV), dq, dk, dv, small)
    torch.cuda.synchronize()
    dq_r, _, _ = OA.attention_bwd(q[torch.as_tensor(rows)], k, v, gr, rows, np.arange(w.seq))
    assert_close(dq, dq_r, TOL_BF16, "bwd8k r1 dQ unsplit")
    assert_close(dq, dq_split, TOL_BF16, "bwd8k r1 dQ unsplit vs split")


def test_bwd8k_pass_calls_match_combined_call(bwd8k):
    # delta, dQ and dK/dV as separate calls give exactly what cpattn_bwd gives (which
    # forms delta inside its dQ pass)
    w, q, k, v, g = bwd8k
    import context_causal_attention_zigzag_amd as C
    rs, rows, gr, dq_c, dk_c, dv_c = run_bwd(q, k, v, g, w.cp, 2)
    o, lse = rs.stream_fwd("owner")
    gd = gr.to(DEV)
    dq, dk, dv, _ = rs.alloc_bwd_buffers()
    desc = rs.desc()
    qb = C.q_block(rs.q, rs.q_idx)
    segs = [s_ for s_, _, _ in rs.segments("owner")]
    delta = torch.empty((rs.q.shape[0], w.hq), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, C.cpattn_bwd_dq_workspace_bytes(desc, qb, segs)), dtype=torch.uint8, device=DEV)
    say("bwd8k pass calls")
    C.cpattn_bwd_delta(desc, o, gd, delta)
    C.cpattn_bwd_dq(desc, qb, segs, lse, delta, gd, dq, ws)
    C.cpattn_bwd_dkdv(desc, qb, segs, lse, delta, gd, dk, dv)
    torch.cuda.synchronize()
    d_ref = (o.double() * gd.double()).sum(-1).float()
    assert_close(delta, d_ref, 1e-3, "bwd8k r2 delta")
    assert torch.equal(dq, dq_c)
    for a, b in zip(dk + dv, dk_c + dv_c):
        assert torch.equal(a, b)
    # the dQ pass that forms D itself, split and unsplit: the same D and dQ bit for bit
    for wsx in (ws, None):
        delta2 = torch.full_like(delta, float("nan"))
        dq2 = torch.empty_like(dq)
        C.cpattn_bwd_dq_delta(desc, qb, segs, o, lse, gd, delta2, dq2, wsx)
        dq3 = torch.empty_like(dq)
        C.cpattn_bwd_dq(desc, qb, segs, lse, delta, gd, dq3, wsx)
        torch.cuda.synchronize()
        assert torch.equal(delta2, delta) and torch.equal(dq2, dq3)


@pytest.mark.parametrize("seq,cp,hq,hkv,d", [(800, 4, 4, 2, 128), (512, 2, 8, 1, 64), (384, 2, 12, 4, 128)])
def test_bwd_small_shapes_and_owner_sums(seq, cp, hq, hkv, d):
    q = workloads.randn((seq, hq, d), 21, "bf16", 0)
    k = workloads.randn((seq, hkv, d), 21, "bf16", 1)
    v = workloads.randn((seq, hkv, d), 21, "bf16", 2)
    g = workloads.randn((seq, hq, d), 21, "bf16", 3)
    dk_sum = torch.zeros((seq, hkv, d), dtype=torch.float64)
    dv_sum = torch.zeros((seq, hkv, d), dtype=torch.float64)
    for r in range(cp):
        rs, dk, dv = check_bwd(f"bwd{seq}", q, k, v, g, cp, r)
        for o_idx, owner in enumerate(ring_order(cp, r)):
            orow = torch.as_tensor(rs.owners[owner].idx.cpu().numpy().astype(np.int64))
            dk_sum[orow] += dk[o_idx].cpu().double()
            dv_sum[orow] += dv[o_idx].cpu().double()
    # contributions of all emulated ranks summed at their owners = full-sequence gradients
    _, dk_f, dv_f = OA.attention_bwd(q, k, v, g)
    assert_close(dk_sum, dk_f, TOL_BF16, f"bwd{seq} owner-summed dK")
    assert_close(dv_sum, dv_f, TOL_BF16, f"bwd{seq} owner-summed dV")


def test_bwd_eight_wave_plans(monkeypatch):
    # plans for 2 compute units: the dQ pass runs its eight-wave work-groups
    monkeypatch.setenv("CPATTN_NUM_CUS", "2")
    q = workloads.randn((800, 4, 128), 24, "bf16", 0)
    k = workloads.randn((800, 2, 128), 24, "bf16", 1)
    v = workloads.randn((800, 2, 128), 24, "bf16", 2)
    g = workloads.randn((800, 4, 128), 24, "bf16", 3)
    for r in range(4):
        check_bwd("bwd8w", q, k, v, g, 4, r)


def test_bwd_packed_small():
    lengths = [8, 64, 136, 0, 16, 256, 8, 32, 520]
    cu = workloads.cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    q = workloads.randn((total, 4, 128), 22, "bf16", 0)
    k = workloads.randn((total, 2, 128), 22, "bf16", 1)
    v = workloads.randn((total, 2, 128), 22, "bf16", 2)
    g = workloads.randn((total, 4, 128), 22, "bf16", 3)
    for r in range(2):
        check_bwd("bwd-packed", q, k, v, g, 2, r, cu)


def test_bwd_packed_ranked_order():
    # eight head groups: the dQ launch orders query tiles by the KV tiles they walk
    lengths = [8, 64, 136, 0, 16, 256, 8, 32, 520, 1024, 40, 4, 300]
    cu = workloads.cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    q = workloads.randn((total, 8, 128), 23, "bf16", 0)
    k = workloads.randn((total, 8, 128), 23, "bf16", 1)
    v = workloads.randn((total, 8, 128), 23, "bf16", 2)
    g = workloads.randn((total, 8, 128), 23, "bf16", 3)
    for r in range(2):
        check_bwd("bwd-ranked", q, k, v, g, 2, r, cu)


def test_bwd_fully_masked_rows_give_zero_gradients():
    import context_causal_attention_zigzag_amd as C
    tq, tk, h, d = 40, 64, 2, 128
    q = workloads.randn((tq, h, d), 23, "bf16", 0).to(DEV)
    k = workloads.randn((tk, h, d), 23, "bf16", 1).to(DEV)
    v = workloads.randn((tk, h, d), 23, "bf16", 2).to(DEV)
    g = workloads.randn((tq, h, d), 23, "bf16", 3).to(DEV)
    qpos = torch.arange(tq, dtype=torch.int32, device=DEV)
    kpos = torch.arange(tk, dtype=torch.int32, device=DEV) + 100
    desc = C.attn_desc(h, h, d)
    o = torch.empty_like(q)
    lse = torch.empty((tq, h), dtype=torch.float32, device=DEV)
    say("bwd fully masked")
    C.cpattn_stream_fwd(desc, C.q_block(q, qpos), [C.kv_seg(k, v, kpos)], o, lse)
    dq = torch.full((tq, h, d), 7.0, device=DEV)
    dk = torch.full((tk, h, d), 7.0, device=DEV)
    dv = torch.full((tk, h, d), 7.0, device=DEV)
    ws = torch.empty(C.cpattn_bwd_workspace_bytes(desc, C.q_block(q, qpos), [C.kv_seg(k, v, kpos)]),
                     dtype=torch.uint8, device=DEV)
    C.cpattn_bwd(desc, C.q_block(q, qpos), [C.kv_seg(k, v, kpos)], o, lse, g, dq, [dk], [dv], ws)
    torch.cuda.synchronize()
    assert torch.all(dq == 0) and torch.all(dk == 0) and torch.all(dv == 0)


@pytest.mark.parametrize("n_keys,n_segs", [(60000, 10), (78000, 20)])
def test_more_tiles_than_the_lds_boundary_table(n_keys, n_segs):
    # The forward's and dQ's boundary searches read a table of every 64-key tile in LDS,
    # 1152 tiles at d = 64: 60000 keys in 10 segments (940 tiles) fit it, 78000 keys in
    # 20 segments (1220 tiles) do not, so the searches read global memory.  Both must
    # match the oracle, forward and backward.
    import context_causal_attention_zigzag_amd as C
    hq, d = 1, 64
    k = workloads.randn((n_keys, hq, d), 31, "bf16", 1)
    v = workloads.randn((n_keys, hq, d), 31, "bf16", 2)
    rng = np.random.default_rng(31)
    qpos = np.sort(rng.choice(n_keys, 300, replace=False)).astype(np.int32)
    q = workloads.randn((300, hq, d), 31, "bf16", 0)
    g = workloads.randn((300, hq, d), 31, "bf16", 3)
    gq, gk, gv, gg = q.to(DEV), k.to(DEV), v.to(DEV), g.to(DEV)
    kpos = torch.arange(n_keys, dtype=torch.int32, device=DEV)
    qp = torch.as_tensor(qpos, device=DEV)
    bounds = np.linspace(0, n_keys, n_segs + 1).astype(int)
    segs = [C.kv_seg(gk[a:b], gv[a:b], kpos[a:b]) for a, b in zip(bounds[:-1], bounds[1:])]
    desc = C.attn_desc(hq, hq, d)
    qb = C.q_block(gq, qp)
    say(f"{n_segs} segments of {n_keys // n_segs} keys: stream forward + backward")
    o = torch.empty_like(gq)
    lse = torch.empty((300, hq), dtype=torch.float32, device=DEV)
    C.cpattn_stream_fwd(desc, qb, segs, o, lse)
    dq = torch.empty((300, hq, d), dtype=torch.float32, device=DEV)
    dk = [torch.empty((b - a, hq, d), dtype=torch.float32, device=DEV) for a, b in zip(bounds[:-1], bounds[1:])]
    dv = [torch.empty_like(x) for x in dk]
    ws = torch.empty(max(1, C.cpattn_bwd_workspace_bytes(desc, qb, segs)), dtype=torch.uint8, device=DEV)
    C.cpattn_bwd(desc, qb, segs, o, lse, gg, dq, dk, dv, ws)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_fwd(q, k, v, qpos, np.arange(n_keys))
    assert_close(o, o_ref, TOL_BF16, f"{n_segs}-seg O")
    dq_r, dk_r, dv_r = OA.attention_bwd(q, k, v, g, qpos, np.arange(n_keys))
    assert_close(dq, dq_r, TOL_BF16, f"{n_segs}-seg dQ")
    assert_close(torch.cat(dk), dk_r, TOL_BF16, f"{n_segs}-seg dK")
    assert_close(torch.cat(dv), dv_r, TOL_BF16, f"{n_segs}-seg dV")
