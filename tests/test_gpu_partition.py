"""Partition kernel vs the oracle: indices and document ids bit-exact, gathers are
exact row copies."""
import numpy as np
import pytest
import torch

import context_causal_attention_zigzag_amd as C
from context_causal_attention_zigzag_amd.rank_share import partition_shard
import oracle
import workloads
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("seq,cp", [(512, 2), (8192, 4), (800, 4), (131072, 8), (64, 1), (48, 3)])
def test_zigzag_indices_and_gather(seq, cp):
    src = torch.arange(seq * 24, dtype=torch.int32).reshape(seq, 3, 8)   # 96-byte rows
    src2 = torch.randn(seq, 4, dtype=torch.float32)                        # 16-byte rows
    g_src, g_src2 = src.to(DEV), src2.to(DEV)
    for r in range(cp):
        say(f"partition zigzag seq={seq} cp={cp} rank={r}")
        sh = partition_shard(C.PART_ZIGZAG, seq, cp, r, [g_src, g_src2])
        torch.cuda.synchronize()
        want = oracle.zigzag_indices(seq, cp, r)
        assert np.array_equal(sh.idx.cpu().numpy(), want)
        assert torch.equal(sh.tensors[0].cpu(), src[torch.as_tensor(want)])
        assert torch.equal(sh.tensors[1].cpu(), src2[torch.as_tensor(want)])


@pytest.mark.parametrize("lengths,cp", [
    (None, 4),                                      # the thd64k mix (seed 4)
    ([8, 64, 136, 0, 16, 256, 8, 32], 2),           # short, ragged, one empty document
    ([4096], 4),                                    # one document = zigzag
])
def test_thd_indices_docs_and_gather(lengths, cp):
    if lengths is None:
        lengths = workloads.thd_lengths(4)
    cu = workloads.cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    cu_dev = torch.as_tensor(cu, dtype=torch.int32, device=DEV)
    src = torch.randn(total, 2, 64).to(torch.bfloat16)
    g_src = src.to(DEV)
    for r in range(cp):
        say(f"partition thd docs={len(lengths)} total={total} cp={cp} rank={r}")
        sh = partition_shard(C.PART_THD, total, cp, r, [g_src], cu.tolist(), cu_dev, with_doc=True)
        torch.cuda.synchronize()
        want = oracle.thd_indices(cu, cp, r)
        assert np.array_equal(sh.idx.cpu().numpy(), want)
        assert np.array_equal(sh.doc.cpu().numpy(), oracle.thd_doc_ids(cu, want))
        assert torch.equal(sh.tensors[0].cpu().view(torch.int16), src[torch.as_tensor(want)].view(torch.int16))


def test_empty_partition_is_noop():
    say("partition total=0")
    idx = torch.empty(0, dtype=torch.int32, device=DEV)
    C.cpattn_partition(C.PART_ZIGZAG, 0, 4, 1, idx)
    torch.cuda.synchronize()


@pytest.mark.parametrize("mode", ["zigzag", "thd"])
def test_indices_only(mode):
    # no tensors to gather: the kernel writes the index (and document) outputs alone,
    # over several blocks of rows
    if mode == "zigzag":
        total, cp, cu, cu_dev = 3000, 4, None, None
    else:
        cu = workloads.cu_seqlens_from_lengths([8, 64, 136, 0, 16, 256, 8, 32, 2040])
        total, cp = int(cu[-1]), 2
        cu_dev = torch.as_tensor(cu, dtype=torch.int32, device=DEV)
    for r in range(cp):
        say(f"partition indices only {mode} total={total} cp={cp} rank={r}")
        idx = torch.empty(total // cp, dtype=torch.int32, device=DEV)
        doc = torch.empty(total // cp, dtype=torch.int32, device=DEV) if cu is not None else None
        C.cpattn_partition(C.PART_THD if cu is not None else C.PART_ZIGZAG, total, cp, r, idx, doc,
                           (), (), None if cu is None else cu.tolist(), cu_dev)
        torch.cuda.synchronize()
        want = oracle.thd_indices(cu, cp, r) if cu is not None else oracle.zigzag_indices(total, cp, r)
        assert np.array_equal(idx.cpu().numpy(), want)
        if cu is not None:
            assert np.array_equal(doc.cpu().numpy(), oracle.thd_doc_ids(cu, want))


@pytest.mark.parametrize("seq,cp", [(512, 2), (8192, 4), (800, 4), (131072, 8), (48, 3), (64, 1), (12, 4)])
def test_striped_indices_and_gather(seq, cp):
    src = torch.arange(seq * 24, dtype=torch.int32).reshape(seq, 3, 8)
    src2 = torch.randn(seq, 4, dtype=torch.float32)
    g_src, g_src2 = src.to(DEV), src2.to(DEV)
    for r in range(cp):
        say(f"partition striped seq={seq} cp={cp} rank={r}")
        sh = partition_shard(C.PART_STRIPED, seq, cp, r, [g_src, g_src2], with_doc=True)
        torch.cuda.synchronize()
        want = oracle.striped_indices(seq, cp, r)
        assert np.array_equal(sh.idx.cpu().numpy(), want)
        assert np.all(sh.doc.cpu().numpy() == 0)
        assert torch.equal(sh.tensors[0].cpu(), src[torch.as_tensor(want)])
        assert torch.equal(sh.tensors[1].cpu(), src2[torch.as_tensor(want)])
