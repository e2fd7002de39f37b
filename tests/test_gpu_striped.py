"""Attention on striped shares (rank r holds tokens r, r + cp, ...): the partition
kernel's striped split feeds the same forward and backward kernels, whose tile
classification reads the positions, so the results must match the oracle's full
attention for the rank's rows exactly as for zigzag shares."""
import numpy as np
import pytest
import torch

from context_causal_attention_zigzag_amd.rank_share import build_rank_share, ring_order
import oracle
from oracle import attention as OA
import workloads
from gpu_common import DEV, TOL_BF16, TOL_LSE_BF16, assert_close, say

pytestmark = pytest.mark.gpu

S, CP, HQ, HKV, D = 4096, 4, 4, 2, 128


@pytest.mark.parametrize("rank", [0, 3])
def test_striped_share_forward_and_backward(rank):
    q = workloads.randn((S, HQ, D), 41, "bf16", 0)
    k = workloads.randn((S, HKV, D), 41, "bf16", 1)
    v = workloads.randn((S, HKV, D), 41, "bf16", 2)
    rows = oracle.striped_indices(S, CP, rank)
    g = workloads.randn((len(rows), HQ, D), 41, "bf16", 3)
    rs = build_rank_share(q.to(DEV), k.to(DEV), v.to(DEV), CP, rank, striped=True)
    assert np.array_equal(rs.q_idx.cpu().numpy(), rows)
    keys = np.arange(S)
    o_ref, l_ref = OA.attention_fwd(q[torch.as_tensor(rows)], k, v, rows, keys)
    for gran in ("owner", "chunk"):
        for ws in ("auto", None):
            tag = f"striped r{rank} {gran}/{'split' if ws else 'nosplit'}"
            say(tag)
            o, lse = rs.stream_fwd(gran, workspace=ws)
            edges, parts = rs.alloc_tile_buffers(gran)
            rs.tile_fwd(edges, parts, workspace=ws)
            o2, l2 = rs.merge(edges, parts)
            torch.cuda.synchronize()
            assert_close(o, o_ref, TOL_BF16, f"{tag} stream O")
            assert_close(lse, l_ref, TOL_LSE_BF16, f"{tag} stream LSE")
            assert_close(o2, o_ref, TOL_BF16, f"{tag} tile O")
            assert_close(l2, l_ref, TOL_LSE_BF16, f"{tag} tile LSE")
    o, lse = rs.stream_fwd("owner")
    dq, dk, dv = rs.bwd(o, lse, g.to(DEV))
    torch.cuda.synchronize()
    dq_r, dk_r, dv_r = OA.attention_bwd(q[torch.as_tensor(rows)], k, v, g, rows, keys)
    assert_close(dq, dq_r, TOL_BF16, f"striped r{rank} dQ")
    for i, owner in enumerate(ring_order(CP, rank)):
        orow = oracle.striped_indices(S, CP, owner)
        assert np.array_equal(rs.owners[owner].idx.cpu().numpy(), orow)
        assert_close(dk[i], dk_r[orow], TOL_BF16, f"striped r{rank} dK owner {owner}")
        assert_close(dv[i], dv_r[orow], TOL_BF16, f"striped r{rank} dV owner {owner}")
