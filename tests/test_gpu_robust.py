"""Failure handling on the GPU: NaN inputs reach the outputs they feed (nothing masks
them away as an empty row), and an auto-sized workspace is safe when the kernels run
on a stream other than the current one.

NaN cases, on one rank of an 8K zigzag share (rank 0 holds positions 0..1023 and
7168..8191; the emulated owners' K/V rows are those of the other ranks):
* a NaN in one query row makes that row's output and log-sum-exp NaN, for every
  forward form, and leaves the other rows as the oracle computes them;
* a NaN in the key or value row at position 2000 makes every row of the heavy chunk
  (which sees position 2000) NaN in O (and, for the key, in the LSE), while the light
  chunk (positions <= 1023, which shares no key tile with position 2000) stays finite
  and equal to the oracle;
* a NaN in the upstream gradient of one row makes that row's dQ NaN and the dK / dV
  rows of the keys it sees NaN, while the dQ of every other row stays finite.
"""
import numpy as np
import pytest
import torch

import context_causal_attention_zigzag_amd as C
from context_causal_attention_zigzag_amd.rank_share import build_rank_share
import oracle
import workloads
from gpu_common import DEV, TOL_BF16, TOL_LSE_BF16, assert_close, oracle_fwd_rows, say

pytestmark = pytest.mark.gpu

SEQ, CP, RANK, HQ, HKV, D = 8192, 4, 0, 2, 1, 128


def inputs():
    q = workloads.randn((SEQ, HQ, D), 12, "bf16", 0)
    k = workloads.randn((SEQ, HKV, D), 12, "bf16", 1)
    v = workloads.randn((SEQ, HKV, D), 12, "bf16", 2)
    return q, k, v


def forwards(rs):
    out = {}
    for gran in ("owner", "chunk"):
        for ws in ("auto", None):
            out[f"stream/{gran}/{'split' if ws else 'nosplit'}"] = rs.stream_fwd(gran, workspace=ws)
            edges, parts = rs.alloc_tile_buffers(gran)
            rs.tile_fwd(edges, parts, workspace=ws)
            out[f"tile/{gran}/{'split' if ws else 'nosplit'}"] = rs.merge(edges, parts)
    torch.cuda.synchronize()
    return out


def test_nan_query_row_propagates_to_its_row_only():
    q, k, v = inputs()
    rows = oracle.zigzag_indices(SEQ, CP, RANK)
    bad_local = 1500                       # a heavy-chunk row
    q[rows[bad_local], 1, 5] = float("nan")
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), CP, RANK)
    sample = np.array([0, 700, 1023, 1024, 1499, 1501, 2047])
    o_ref, l_ref = oracle_fwd_rows(q, k, v, rows[sample])
    for name, (o, lse) in forwards(rs).items():
        say(f"NaN in q row: {name}")
        assert torch.isnan(o[bad_local, 1]).all() and torch.isnan(lse[bad_local, 1])
        assert torch.isfinite(o[bad_local, 0]).all() and torch.isfinite(lse[bad_local, 0])
        assert int(torch.isnan(o).sum()) == D and int(torch.isnan(lse).sum()) == 1
        li = torch.as_tensor(sample, device=DEV)
        assert_close(o[li], o_ref, TOL_BF16, f"{name} other rows O")
        assert_close(lse[li], l_ref, TOL_LSE_BF16, f"{name} other rows LSE")


@pytest.mark.parametrize("which", ["k", "v"])
def test_nan_key_or_value_reaches_every_row_that_sees_it(which):
    q, k, v = inputs()
    (k if which == "k" else v)[2000, 0, :] = float("nan")
    rows = oracle.zigzag_indices(SEQ, CP, RANK)
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), CP, RANK)
    light = np.arange(0, 1024, 97)
    o_ref, l_ref = oracle_fwd_rows(q, k, v, rows[light])
    for name, (o, lse) in forwards(rs).items():
        say(f"NaN in {which} row 2000: {name}")
        assert torch.isnan(o[1024:]).all(), "every heavy-chunk row sees key 2000"
        if which == "k":
            assert torch.isnan(lse[1024:]).all()
        else:
            assert torch.isfinite(lse).all()
        assert torch.isfinite(o[:1024]).all() and torch.isfinite(lse[:1024]).all()
        li = torch.as_tensor(light, device=DEV)
        assert_close(o[li], o_ref, TOL_BF16, f"{name} light chunk O")
        assert_close(lse[li], l_ref, TOL_LSE_BF16, f"{name} light chunk LSE")


def test_nan_upstream_gradient_row():
    q, k, v = inputs()
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), CP, RANK)
    n = SEQ // CP
    g = workloads.randn((n, HQ, D), 13, "bf16", 3)
    bad_local = 100                        # position 100 in the light chunk
    g[bad_local, 0, 7] = float("nan")
    o, lse = rs.stream_fwd("owner")
    dq, dk, dv = rs.bwd(o, lse, g.to(DEV))
    torch.cuda.synchronize()
    assert torch.isnan(dq[bad_local, 0]).any()
    others = torch.ones(n, dtype=torch.bool)
    others[bad_local] = False
    assert torch.isfinite(dq[others.to(DEV)]).all()
    assert torch.isfinite(dq[bad_local, 1]).all()
    # owner 0 (the rank itself, first segment) holds positions 0..1023 first: keys
    # 0..100 are seen by the bad row
    assert torch.isnan(dv[0][:101, 0, 7]).all()
    assert torch.isnan(dk[0][:101, 0]).any(dim=-1).all()
    # keys at positions >= 1024 never meet the light chunk's rows: finite
    for s_dk, s_dv, (seg, (owner, part), (a, b)) in zip(dk, dv, rs.segments("owner")):
        pos = rs.owners[owner].idx[a:b]
        far = pos >= 1024
        assert torch.isfinite(s_dk[far]).all() and torch.isfinite(s_dv[far]).all()


def test_auto_workspace_on_a_side_stream():
    q, k, v = inputs()
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), CP, RANK)
    o_ref, l_ref = rs.stream_fwd("owner")
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    o = torch.empty_like(o_ref)
    lse = torch.empty_like(l_ref)
    desc = rs.desc()
    segs = [s_ for s_, _, _ in rs.segments("owner")]
    qb = C.q_block(rs.q, rs.q_idx, rs.q_doc)
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        C.cpattn_stream_fwd(desc, qb, segs, o, lse, workspace="auto", stream=side)
        # the current stream allocates and scribbles while the side stream still runs
        junk = torch.full((64 << 20,), 7, dtype=torch.uint8, device=DEV)
        del junk
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, l_ref)
