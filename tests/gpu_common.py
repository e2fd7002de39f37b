"""Shared pieces of the GPU parity tests: run a rank share through the C ABI, compute
the oracle's answer for the same rows on the CPU, compare."""
import sys

import numpy as np
import torch

import oracle
from oracle import attention as OA

DEV = "cuda"

# tolerances fixed for this path: fp32 inputs 1e-5 max abs; bf16 inputs with fp32
# accumulation 2e-2 max abs on O and gradients, 1e-3 on the log-sum-exp
TOL_F32 = 1e-5
TOL_BF16 = 2e-2
TOL_LSE_BF16 = 1e-3


def say(msg):
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def np64(t):
    if isinstance(t, np.ndarray):
        return t.astype(np.float64)
    return t.detach().to("cpu").float().double().numpy()


def max_abs(gpu, ref):
    g, r = np64(gpu), np64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    gi, ri = np.isneginf(g), np.isneginf(r)
    assert np.array_equal(gi, ri), "-inf pattern differs"
    assert not np.any(np.isnan(g)), "NaN in GPU output"
    fin = ~ri
    return float(np.max(np.abs(g[fin] - r[fin]))) if np.any(fin) else 0.0


def assert_close(gpu, ref, tol, what):
    err = max_abs(gpu, ref)
    say(f"{what}: max abs err {err:.3e} (tol {tol:g})")
    assert err <= tol, f"{what}: max abs err {err} > {tol}"


def rank_rows(seq, cp, rank, cu=None):
    if cu is None:
        return oracle.zigzag_indices(seq, cp, rank), None
    rows = oracle.thd_indices(cu, cp, rank)
    return rows, oracle.thd_doc_ids(cu, rows)


def oracle_fwd_rows(q, k, v, rows, cu=None, all_docs=None):
    """Oracle (O, LSE) of the queries at global rows `rows` against the whole sequence."""
    seq = k.shape[0]
    tq = q[torch.as_tensor(rows)]
    if cu is None:
        return OA.attention_fwd(tq, k, v, rows, np.arange(seq))
    qdoc = oracle.thd_doc_ids(cu, rows)
    return OA.attention_fwd(tq, k, v, rows, np.arange(seq), qdoc, all_docs, OA.MASK_CAUSAL_DOC)
