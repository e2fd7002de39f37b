"""Rotary embedding fused into the partition gather, against the oracle.

For every split (zigzag, striped, packed documents) the rotated tensors must equal
the oracle's rotation of the rows the rank keeps at their true positions (global,
or inside the document), the copied tensors and the index / document outputs must
be bit-exact.  Bounds: fp32 1e-5 max abs; bf16 2e-2 max abs and, derived from the
arithmetic, within one rounding of the exact value: |gpu - ref| <= 2^-8 |ref| + 4e-6
(the fp32 rotation with fp32 cos/sin is good to ~1e-6; rounding to bf16 moves a
value by at most 2^-8 of itself)."""
import numpy as np
import pytest
import torch

import context_causal_attention_zigzag_amd as C
import oracle
from oracle import rope as R
import workloads
from gpu_common import DEV, np64, say

pytestmark = pytest.mark.gpu


def rows_and_positions(mode, total, cp, rank, cu):
    if mode == C.PART_ZIGZAG:
        rows = oracle.zigzag_indices(total, cp, rank)
        return rows, rows
    if mode == C.PART_STRIPED:
        rows = oracle.striped_indices(total, cp, rank)
        return rows, rows
    rows = oracle.thd_indices(cu, cp, rank)
    return rows, R.thd_positions(cu, rows)


def check_rotated(gpu, x, pos, base, interleaved, what):
    ref = R.apply_rope(x, pos, base, interleaved)
    g = np64(gpu)
    err = np.abs(g - ref)
    say(f"{what}: max abs err {float(err.max()):.3e}")
    if gpu.dtype == torch.float32:
        assert float(err.max()) <= 1e-5, what
    else:
        assert float(err.max()) <= 2e-2, what
        assert np.all(err <= 2.0 ** -8 * np.abs(ref) + 4e-6), f"{what}: beyond one bf16 rounding"


CASES = [
    # name, mode, total, cp, ranks, q heads, k heads, d, dtype, interleaved, base
    ("zigzag8k", C.PART_ZIGZAG, 8192, 4, (0, 1, 2, 3), 8, 2, 128, torch.bfloat16, False, 10000.0),
    ("zigzag128k", C.PART_ZIGZAG, 131072, 8, (0, 7), 32, 8, 128, torch.bfloat16, False, 10000.0),
    ("striped8k-f32-il", C.PART_STRIPED, 8192, 4, (0, 3), 4, 1, 64, torch.float32, True, 500000.0),
    ("thd64k", C.PART_THD, None, 4, (1,), 16, 16, 128, torch.bfloat16, False, 10000.0),
    ("thd-ragged-il", C.PART_THD, [8, 64, 136, 0, 16, 256, 8, 32], 2, (0, 1), 2, 1, 256, torch.bfloat16, True,
     10000.0),
    ("zigzag-d16-f32", C.PART_ZIGZAG, 960, 3, (0, 2), 1, 1, 16, torch.float32, False, 10000.0),
    ("zigzag-d16-bf16-il", C.PART_ZIGZAG, 960, 3, (1,), 1, 3, 16, torch.bfloat16, True, 0.0),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_rope_in_partition(case):
    name, mode, total, cp, ranks, hq, hk, d, dt, il, base = case
    cu = cu_dev = None
    if mode == C.PART_THD:
        lengths = workloads.thd_lengths(4) if total is None else total
        cu = workloads.cu_seqlens_from_lengths(lengths)
        total = int(cu[-1])
        cu_dev = torch.as_tensor(cu, dtype=torch.int32, device=DEV)
    q = workloads.randn((total, hq, d), 21, "f32" if dt == torch.float32 else "bf16", 0)
    k = workloads.randn((total, hk, d), 21, "f32" if dt == torch.float32 else "bf16", 1)
    v = workloads.randn((total, hk, d), 21, "bf16", 2)
    gq, gk, gv = q.to(DEV), k.to(DEV), v.to(DEV)
    rope = C.rope_desc((0, 1), dt, d, il, base)
    eff_base = base if base > 0 else 10000.0
    n = total // cp
    for r in ranks:
        say(f"rope {name} rank={r}")
        idx = torch.empty(n, dtype=torch.int32, device=DEV)
        doc = torch.empty(n, dtype=torch.int32, device=DEV)
        outs = [torch.empty((n,) + tuple(t.shape[1:]), dtype=t.dtype, device=DEV) for t in (gq, gk, gv)]
        C.cpattn_partition(mode, total, cp, r, idx, doc, [gq, gk, gv], outs, None if cu is None else cu.tolist(),
                           cu_dev, rope=rope)
        torch.cuda.synchronize()
        rows, pos = rows_and_positions(mode, total, cp, r, cu)
        assert np.array_equal(idx.cpu().numpy(), rows)
        if cu is not None:
            assert np.array_equal(doc.cpu().numpy(), oracle.thd_doc_ids(cu, rows))
        ri = torch.as_tensor(rows)
        check_rotated(outs[0], q[ri], pos, eff_base, il, f"{name} r{r} Q")
        check_rotated(outs[1], k[ri], pos, eff_base, il, f"{name} r{r} K")
        assert torch.equal(outs[2].cpu().view(torch.int16), v[ri].view(torch.int16)), "V is copied unchanged"


def test_rope_every_tensor_rotated_and_indices():
    # tensor 0 rotated and no plain tensor: the rotation kernel alone writes the indices
    total, cp, r, d = 4096, 4, 2, 128
    q = workloads.randn((total, 2, d), 22, "bf16", 0)
    gq = q.to(DEV)
    idx = torch.empty(total // cp, dtype=torch.int32, device=DEV)
    out = torch.empty((total // cp, 2, d), dtype=torch.bfloat16, device=DEV)
    C.cpattn_partition(C.PART_ZIGZAG, total, cp, r, idx, None, [gq], [out], rope=C.rope_desc((0,), torch.bfloat16, d))
    torch.cuda.synchronize()
    rows = oracle.zigzag_indices(total, cp, r)
    assert np.array_equal(idx.cpu().numpy(), rows)
    check_rotated(out, q[torch.as_tensor(rows)], rows, 10000.0, False, "Q only")


def test_rope_after_the_split_equals_rotating_the_full_sequence():
    # the split of the pages' checklist: rotating after the split at the kept rows'
    # positions equals rotating the full sequence, so attention on a rank's rotated
    # rows equals full-sequence attention on rotated inputs for those rows
    total, cp, r, hq, hk, d = 2048, 4, 1, 2, 1, 128
    q = workloads.randn((total, hq, d), 23, "bf16", 0)
    k = workloads.randn((total, hk, d), 23, "bf16", 1)
    n = total // cp
    rope = C.rope_desc((0, 1), torch.bfloat16, d)
    idx = torch.empty(n, dtype=torch.int32, device=DEV)
    outs = [torch.empty((n, h, d), dtype=torch.bfloat16, device=DEV) for h in (hq, hk)]
    C.cpattn_partition(C.PART_ZIGZAG, total, cp, r, idx, None, [q.to(DEV), k.to(DEV)], outs, rope=rope)
    torch.cuda.synchronize()
    rows = oracle.zigzag_indices(total, cp, r)
    full_q = R.apply_rope(q, np.arange(total))
    full_k = R.apply_rope(k, np.arange(total))
    check_rotated(outs[0], q[torch.as_tensor(rows)], rows, 10000.0, False, "Q rows")
    assert np.max(np.abs(np64(outs[1]) - full_k[rows])) <= 2e-2
    assert np.max(np.abs(np64(outs[0]) - full_q[rows])) <= 2e-2
