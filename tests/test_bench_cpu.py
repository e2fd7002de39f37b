"""The benchmark's host-side contract: one-GPU refusal and its visible-pair counts."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

import oracle
from oracle import attention as OA
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


@pytest.mark.parametrize("lengths,cp,rank", [([8, 64, 136, 0, 16, 256, 8, 32], 2, 1), ([48, 16, 96], 4, 2)])
def test_packed_pair_count_matches_brute_force(lengths, cp, rank):
    # bench.py counts a packed share's visible pairs per local row as its position minus
    # its document's start, plus one; count them here from the mask itself
    cu = workloads.cu_seqlens_from_lengths(lengths)
    total = int(cu[-1])
    rows = oracle.thd_indices(cu, cp, rank)
    docs = oracle.thd_doc_ids(cu, rows)
    per_row = int(np.sum(rows - np.asarray(cu, dtype=np.int64)[docs] + 1))
    keys = np.arange(total)
    vis = OA.visible_mask(rows, keys, docs, oracle.thd_doc_ids(cu, keys), OA.MASK_CAUSAL_DOC)
    assert per_row == int(vis.sum())


@pytest.mark.parametrize("seq,cp", [(512, 2), (8192, 4), (96, 3)])
def test_zigzag_pair_count_matches_brute_force(seq, cp):
    # bench.py uses S(S+1)/(2cp) for every zigzag rank
    keys = np.arange(seq)
    for rank in range(cp):
        rows = oracle.zigzag_indices(seq, cp, rank)
        vis = OA.visible_mask(rows, keys)
        assert int(vis.sum()) == seq * (seq + 1) // (2 * cp)
