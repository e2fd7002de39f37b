"""Forward parity on the GPU: streaming form and tile + merge form vs the oracle.

Full element-by-element comparisons on the tiny (fp32) and s8k (bf16, all four ranks)
workloads and on small shapes that exercise ragged tiles, grouped queries, d=64,
packed documents, fully masked rows, long segment / edge lists and the no-mask case.
"""
import numpy as np
import pytest
import torch

import context_causal_attention_zigzag_amd as C
from context_causal_attention_zigzag_amd.rank_share import build_rank_share
import oracle
from oracle import attention as OA
import workloads
from gpu_common import (DEV, TOL_BF16, TOL_F32, TOL_LSE_BF16, assert_close, oracle_fwd_rows,
                        rank_rows, say)

pytestmark = pytest.mark.gpu


def check_share(name, q, k, v, cp, rank, cu=None, granularities=("owner", "chunk"), tile=True):
    f32 = q.dtype == torch.float32
    tol_o, tol_l = (TOL_F32, TOL_F32) if f32 else (TOL_BF16, TOL_LSE_BF16)
    rows, _ = rank_rows(q.shape[0], cp, rank, cu)
    all_docs = None if cu is None else oracle.thd_doc_ids(cu, np.arange(q.shape[0]))
    o_ref, l_ref = oracle_fwd_rows(q, k, v, rows, cu, all_docs)
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), cp, rank, cu)
    assert np.array_equal(rs.q_idx.cpu().numpy(), rows)
    for gran in granularities:
        # "auto": KV splits over several work-groups where planned; None: one per query tile
        for ws in ("auto", None):
            tag = "split" if ws else "nosplit"
            say(f"{name} rank={rank} stream gran={gran} {tag}")
            o, lse = rs.stream_fwd(gran, workspace=ws)
            torch.cuda.synchronize()
            assert_close(o, o_ref, tol_o, f"{name} r{rank} stream/{gran}/{tag} O")
            assert_close(lse, l_ref, tol_l, f"{name} r{rank} stream/{gran}/{tag} LSE")
            if tile:
                say(f"{name} rank={rank} tile+merge gran={gran} {tag}")
                edges, parts = rs.alloc_tile_buffers(gran)
                rs.tile_fwd(edges, parts, workspace=ws)
                o2, l2 = rs.merge(edges, parts)
                torch.cuda.synchronize()
                assert_close(o2, o_ref, tol_o, f"{name} r{rank} tile/{gran}/{tag} O")
                assert_close(l2, l_ref, tol_l, f"{name} r{rank} tile/{gran}/{tag} LSE")
    return rs


def test_tiny_fp32_both_ranks():
    w = workloads.WORKLOADS["tiny"]
    q, k, v = workloads.full_qkv(w)
    for r in w.ranks:
        check_share("tiny", q, k, v, w.cp, r)


@pytest.fixture(scope="module")
def s8k():
    w = workloads.WORKLOADS["s8k"]
    return w, workloads.full_qkv(w)


@pytest.mark.parametrize("rank", [0, 1, 2, 3])
def test_s8k_rank(s8k, rank):
    w, (q, k, v) = s8k
    check_share("s8k", q, k, v, w.cp, rank, granularities=("owner",))


@pytest.mark.parametrize("seq,cp,hq,hkv,d,dtype", [
    (800, 4, 4, 2, 128, "bf16"),      # 100-row chunks: ragged query and key tiles, GQA group 2
    (512, 2, 8, 1, 64, "bf16"),       # d=64, one kv head for 8 query heads
    (384, 2, 12, 4, 128, "bf16"),     # group 3
    (256, 2, 2, 2, 128, "f32"),       # fp32 with d=128
    (72, 3, 2, 1, 64, "f32"),         # 12-row chunks
])
def test_small_shapes(seq, cp, hq, hkv, d, dtype):
    q = workloads.randn((seq, hq, d), 11, dtype, 0)
    k = workloads.randn((seq, hkv, d), 11, dtype, 1)
    v = workloads.randn((seq, hkv, d), 11, dtype, 2)
    for r in range(cp):
        check_share(f"small{seq}x{hq}/{hkv}x{d}{dtype}", q, k, v, cp, r)


@pytest.fixture
def few_cus(monkeypatch):
    """Plans computed for 2 compute units: query tiles alone fill them, so the bf16
    kernels run their eight-wave work-groups (the ping-pong forward step) on small shapes."""
    monkeypatch.setenv("CPATTN_NUM_CUS", "2")


@pytest.mark.parametrize("seq,cp,hq,hkv,d", [
    (800, 4, 4, 2, 128),   # ragged query and key tiles, GQA group 2
    (512, 2, 8, 1, 64),    # d=64, 8 query heads on one kv head
    (384, 2, 12, 4, 128),  # group 3
])
def test_small_shapes_eight_wave(few_cus, seq, cp, hq, hkv, d):
    q = workloads.randn((seq, hq, d), 14, "bf16", 0)
    k = workloads.randn((seq, hkv, d), 14, "bf16", 1)
    v = workloads.randn((seq, hkv, d), 14, "bf16", 2)
    for r in range(cp):
        check_share(f"small8w{seq}x{hq}/{hkv}x{d}", q, k, v, cp, r)


def test_packed_documents_eight_wave(few_cus):
    lengths = [8, 64, 136, 0, 16, 256, 8, 32, 520]
    cu = workloads.cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    q = workloads.randn((total, 4, 128), 15, "bf16", 0)
    k = workloads.randn((total, 2, 128), 15, "bf16", 1)
    v = workloads.randn((total, 2, 128), 15, "bf16", 2)
    for r in range(2):
        check_share("packed8w", q, k, v, 2, r, cu=cu, granularities=("owner",))


# Head groups divisible by 8 with the document mask: the bf16 launches order the query
# tiles by the KV tiles their work-groups walk (each XCD takes a block of head groups
# of every job).  Documents of mixed lengths, ragged against the 64-key and 128/256-row
# tiles, and an empty one.
RANKED_LENGTHS = [8, 64, 136, 0, 16, 256, 8, 32, 520, 1024, 40, 4, 300]


@pytest.mark.parametrize("hq,hkv,d", [(8, 8, 128), (16, 8, 64), (16, 16, 128)])
def test_packed_documents_ranked_order(hq, hkv, d):
    cu = workloads.cu_seqlens_from_lengths(RANKED_LENGTHS)
    total = int(cu[-1])
    q = workloads.randn((total, hq, d), 16, "bf16", 0)
    k = workloads.randn((total, hkv, d), 16, "bf16", 1)
    v = workloads.randn((total, hkv, d), 16, "bf16", 2)
    for r in range(2):
        check_share(f"ranked{hq}/{hkv}x{d}", q, k, v, 2, r, cu=cu, granularities=("owner", "chunk"))


def test_packed_documents_ranked_order_eight_wave(few_cus):
    cu = workloads.cu_seqlens_from_lengths(RANKED_LENGTHS)
    total = int(cu[-1])
    q = workloads.randn((total, 8, 128), 17, "bf16", 0)
    k = workloads.randn((total, 8, 128), 17, "bf16", 1)
    v = workloads.randn((total, 8, 128), 17, "bf16", 2)
    for r in range(2):
        check_share("ranked8w", q, k, v, 2, r, cu=cu, granularities=("owner",))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_packed_documents_small(dtype):
    lengths = [8, 64, 136, 0, 16, 256, 8, 32, 520]
    cu = workloads.cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    q = workloads.randn((total, 4, 128), 12, dtype, 0)
    k = workloads.randn((total, 2, 128), 12, dtype, 1)
    v = workloads.randn((total, 2, 128), 12, dtype, 2)
    for r in range(2):
        check_share(f"packed-{dtype}", q, k, v, 2, r, cu=cu, granularities=("owner",))


def _plain_call(q, k, v, qpos, kpos, mask, hq, hkv, d, dtype):
    desc = C.attn_desc(hq, hkv, d, q.dtype, mask)
    o = torch.empty_like(q)
    lse = torch.empty((q.shape[0], hq), dtype=torch.float32, device=DEV)
    C.cpattn_stream_fwd(desc, C.q_block(q, qpos), [C.kv_seg(k, v, kpos)], o, lse)
    return o, lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_fully_masked_rows_and_no_mask(dtype):
    tq, tk, hq, d = 70, 100, 2, 128
    q = workloads.randn((tq, hq, d), 13, dtype, 0)
    k = workloads.randn((tk, hq, d), 13, dtype, 1)
    v = workloads.randn((tk, hq, d), 13, dtype, 2)
    qpos = np.arange(tq) + 40          # rows at positions < 1000 see none of the keys below
    kpos = np.arange(tk) + 1000
    say(f"fully masked rows {dtype}")
    o, lse = _plain_call(q.to(DEV), k.to(DEV), v.to(DEV), torch.as_tensor(qpos, dtype=torch.int32, device=DEV),
                         torch.as_tensor(kpos, dtype=torch.int32, device=DEV), C.MASK_CAUSAL, hq, hq, d, dtype)
    torch.cuda.synchronize()
    assert torch.all(o.float().cpu() == 0) and torch.all(torch.isneginf(lse.cpu()))
    say(f"no mask {dtype}")
    o, lse = _plain_call(q.to(DEV), k.to(DEV), v.to(DEV), torch.as_tensor(qpos, dtype=torch.int32, device=DEV),
                         torch.as_tensor(kpos, dtype=torch.int32, device=DEV), C.MASK_NONE, hq, hq, d, dtype)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_fwd(q, k, v, qpos, kpos, mask=OA.MASK_NONE)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16
    assert_close(o, o_ref, tol, "no-mask O")
    assert_close(lse, l_ref, TOL_F32 if dtype == "f32" else TOL_LSE_BF16, "no-mask LSE")


def test_many_segments_and_edges():
    # 32 unequal segments in a shuffled arrival order; 30 edges (more than one launch)
    seq, hq, d = 1024, 2, 128
    q = workloads.randn((seq, hq, d), 14, "bf16", 0)
    k = workloads.randn((seq, hq, d), 14, "bf16", 1)
    v = workloads.randn((seq, hq, d), 14, "bf16", 2)
    rng = np.random.default_rng(0)
    cuts = np.sort(rng.choice(np.arange(1, seq), 31, replace=False))
    bounds = np.concatenate([[0], cuts, [seq]])
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    pos = torch.arange(seq, dtype=torch.int32, device=DEV)
    order = rng.permutation(32)
    segs = [C.kv_seg(gk[bounds[i]:bounds[i + 1]], gv[bounds[i]:bounds[i + 1]], pos[bounds[i]:bounds[i + 1]])
            for i in order]
    desc = C.attn_desc(hq, hq, d)
    o = torch.empty_like(gq)
    lse = torch.empty((seq, hq), dtype=torch.float32, device=DEV)
    say("32 segments stream")
    C.cpattn_stream_fwd(desc, C.q_block(gq, pos), segs, o, lse)
    torch.cuda.synchronize()
    o_ref, l_ref = OA.attention_fwd(q, k, v)
    assert_close(o, o_ref, TOL_BF16, "32-seg O")
    assert_close(lse, l_ref, TOL_LSE_BF16, "32-seg LSE")
    # 30 edges: 3 query blocks x 10 segments, merged per block
    qb_bounds = [0, 300, 700, seq]
    sb = np.linspace(0, seq, 11).astype(int)
    edges, outs = [], []
    for i in range(3):
        a, b = qb_bounds[i], qb_bounds[i + 1]
        for j in range(10):
            c0, c1 = sb[j], sb[j + 1]
            edges.append((C.q_block(gq[a:b], pos[a:b]), C.kv_seg(gk[c0:c1], gv[c0:c1], pos[c0:c1]), i))
            outs.append((torch.empty((b - a, hq, d), dtype=torch.float32, device=DEV),
                         torch.empty((b - a, hq), dtype=torch.float32, device=DEV)))
    say("30 edges tile")
    C.cpattn_tile_fwd(desc, [e[0] for e in edges], [e[1] for e in edges], [x[0] for x in outs], [x[1] for x in outs])
    o2 = torch.empty_like(gq)
    l2 = torch.empty_like(lse)
    for i in range(3):
        a, b = qb_bounds[i], qb_bounds[i + 1]
        mine = [x for e, x in zip(edges, outs) if e[2] == i]
        C.cpattn_merge([x[0] for x in mine], [x[1] for x in mine], o2[a:b], l2[a:b])
    torch.cuda.synchronize()
    assert_close(o2, o_ref, TOL_BF16, "30-edge O")
    assert_close(l2, l_ref, TOL_LSE_BF16, "30-edge LSE")


def test_merge_groups_match_single_merges():
    # groups of different row counts and part counts, one empty; 11 groups of up to 7 parts
    # take more than one launch (8 groups / 64 parts per launch).  Each group's result must
    # be bit-identical to cpattn_merge on that group alone, and match the oracle's merge.
    rng = np.random.default_rng(9)
    hq, d = 3, 128
    shapes = [(77, 5), (0, 2), (33, 1), (64, 7), (5, 3), (40, 6), (1, 1), (90, 7), (12, 4), (50, 7), (7, 2)]
    for dt in (torch.float32, torch.bfloat16):
        say(f"merge groups {dt}")
        groups, single, refs = [], [], []
        for rows, n in shapes:
            os_ = [rng.standard_normal((rows, hq, d)).astype(np.float32) for _ in range(n)]
            ls_ = [(rng.standard_normal((rows, hq)) * 4).astype(np.float32) for _ in range(n)]
            if rows > 3:
                ls_[0][2, :] = -np.inf
                for j in range(n):
                    ls_[j][3, 1] = -np.inf    # a row empty in every part
            op = [torch.from_numpy(x).to(DEV) for x in os_]
            lp = [torch.from_numpy(x).to(DEV) for x in ls_]
            o = torch.empty((rows, hq, d), dtype=dt, device=DEV)
            lse = torch.empty((rows, hq), dtype=torch.float32, device=DEV)
            groups.append((op, lp, o, lse))
            o1, l1 = torch.empty_like(o), torch.empty_like(lse)
            if rows:
                C.cpattn_merge(op, lp, o1, l1)
            single.append((o1, l1))
            refs.append(OA.merge(list(zip(os_, ls_))) if rows else None)
        C.cpattn_merge_groups(groups)
        torch.cuda.synchronize()
        for (op, lp, o, lse), (o1, l1), ref in zip(groups, single, refs):
            if ref is None:
                continue
            assert torch.equal(o, o1) and torch.equal(lse, l1)
            assert_close(o, ref[0], 1e-5 if dt == torch.float32 else TOL_BF16, f"grouped merge O {dt}")
            assert_close(lse, ref[1], 1e-5, f"grouped merge LSE {dt}")


def test_merge_kernel_against_oracle_merge():
    rng = np.random.default_rng(5)
    n, rows, hq, d = 5, 77, 3, 128
    os_ = [rng.standard_normal((rows, hq, d)).astype(np.float32) for _ in range(n)]
    ls_ = [(rng.standard_normal((rows, hq)) * 4).astype(np.float32) for _ in range(n)]
    ls_[1][3, :] = -np.inf
    for j in range(n):
        ls_[j][10, 1] = -np.inf            # a row empty in every part
    o_ref, l_ref = OA.merge(list(zip(os_, ls_)))
    for dt, tol in ((torch.float32, 1e-5), (torch.bfloat16, TOL_BF16)):
        say(f"merge {dt}")
        o = torch.empty((rows, hq, d), dtype=dt, device=DEV)
        lse = torch.empty((rows, hq), dtype=torch.float32, device=DEV)
        C.cpattn_merge([torch.from_numpy(x).to(DEV) for x in os_], [torch.from_numpy(x).to(DEV) for x in ls_], o, lse)
        torch.cuda.synchronize()
        assert_close(o, o_ref, tol, f"merge O {dt}")
        assert_close(lse, l_ref, 1e-5, f"merge LSE {dt}")


def test_empty_query_block_is_noop_and_deterministic():
    w = workloads.WORKLOADS["s8k"]
    q = workloads.randn((1024, 8, 128), 15, "bf16", 0).to(DEV)
    k = workloads.randn((1024, 8, 128), 15, "bf16", 1).to(DEV)
    v = workloads.randn((1024, 8, 128), 15, "bf16", 2).to(DEV)
    pos = torch.arange(1024, dtype=torch.int32, device=DEV)
    desc = C.attn_desc(8, 8, 128)
    say("empty query block")
    C.cpattn_stream_fwd(desc, C.q_block(q[:0], pos[:0]), [C.kv_seg(k, v, pos)], None, None)
    say("determinism")
    outs = []
    for _ in range(2):
        o = torch.empty_like(q)
        lse = torch.empty((1024, 8), dtype=torch.float32, device=DEV)
        C.cpattn_stream_fwd(desc, C.q_block(q, pos), [C.kv_seg(k, v, pos)], o, lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
