"""The backward entry point for callers that cannot allocate (cpattn_bwd_noalloc, whose
workspace is the library's per-device scratch array) against cpattn_bwd with a
caller workspace, through the C ABI: two calls in a row, the second on a smaller
share, and then the larger one again.  With a scratch array large enough for the
split plan both run the same kernels in the same plan, so the outputs are equal bit
for bit (the bar of the bf16 path would be 2e-2)."""
import pytest
import torch

import context_causal_attention_zigzag_amd as C
from context_causal_attention_zigzag_amd.rank_share import build_rank_share
import workloads
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu

SHAPES = [(8192, 4, 0, 8, 8), (2048, 4, 3, 4, 2), (8192, 4, 0, 8, 8)]


def share(seq, cp, rank, hq, hkv, seed):
    q = workloads.randn((seq, hq, 128), seed, "bf16", 0).to(DEV)
    k = workloads.randn((seq, hkv, 128), seed, "bf16", 1).to(DEV)
    v = workloads.randn((seq, hkv, 128), seed, "bf16", 2).to(DEV)
    rs = build_rank_share(q, k, v, cp, rank)
    g = workloads.randn((seq // cp, hq, 128), seed, "bf16", 3).to(DEV)
    o, lse = rs.stream_fwd("owner")
    return rs, g, o, lse


def test_bwd_noalloc_matches_bwd_on_consecutive_calls():
    assert C.lib.cpattn_bwd_noalloc is not None
    for i, (seq, cp, rank, hq, hkv) in enumerate(SHAPES):
        say(f"noalloc call {i}: S={seq} cp={cp} rank={rank} hq={hq} hkv={hkv}")
        rs, g, o, lse = share(seq, cp, rank, hq, hkv, 30 + i)
        desc = rs.desc()
        qb = C.q_block(rs.q, rs.q_idx, rs.q_doc)
        segs = [s_ for s_, _, _ in rs.segments("owner")]
        ref = rs.bwd(o, lse, g)
        dq, dk, dv, _ = rs.alloc_bwd_buffers("owner")
        for t in [dq] + dk + dv:
            t.fill_(float("nan"))
        C.cpattn_bwd_noalloc(desc, qb, segs, o, lse, g, dq, dk, dv)
        torch.cuda.synchronize()
        assert torch.equal(dq, ref[0]), f"call {i}: dQ differs"
        for s in range(len(segs)):
            assert torch.equal(dk[s], ref[1][s]) and torch.equal(dv[s], ref[2][s]), f"call {i}: segment {s}"
        say(f"noalloc call {i}: equal to cpattn_bwd")
