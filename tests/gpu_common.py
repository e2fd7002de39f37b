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


def assert_close_rows(gpu, ref, tol, rel, what, zero_exact=False):
    """The absolute bound on every element, and per row (the last axis) the error
    relative to that row's largest reference magnitude.  At long context an output
    row is an average over ~1e5 values and its entries are ~1e-3, far below the
    absolute bound; the relative bound is what separates a right row from a row of
    the wrong query, head or key (relative error ~1).  Rows whose reference is zero
    get the absolute bound only, or must be exactly zero with ``zero_exact`` (the K/V
    gradient of a key no query sees: no term reaches it)."""
    g, r = np64(gpu), np64(ref)
    assert g.shape == r.shape, (g.shape, r.shape)
    assert not np.any(np.isnan(g)), f"{what}: NaN in GPU output"
    err = np.abs(g - r)
    mag = np.max(np.abs(r), axis=-1, keepdims=True)
    live = mag[..., 0] > 0
    rel_err = float(np.max(np.max(err, axis=-1)[live] / mag[..., 0][live])) if np.any(live) else 0.0
    abs_err = float(np.max(err)) if err.size else 0.0
    dead = float(np.max(err[~live])) if np.any(~live) else 0.0
    say(f"{what}: max abs err {abs_err:.3e} (tol {tol:g}), max row-relative err {rel_err:.3e} "
        f"(tol {rel:g}), rows {int(np.prod(r.shape[:-1]))}")
    assert abs_err <= tol, f"{what}: max abs err {abs_err} > {tol}"
    assert rel_err <= rel, f"{what}: max row-relative err {rel_err} > {rel}"
    if zero_exact:
        assert dead == 0.0, f"{what}: rows whose reference is zero differ by {dead}"


def oracle_in_threads(fn, n, chunk, what):
    """fn(i0, i1) over [0, n) in chunks, on threads (numpy and BLAS release the GIL),
    BLAS limited to one thread per call; returns the results in order."""
    import os
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    starts = list(range(0, n, chunk))
    done = [0]

    def run(i0):
        out = fn(i0, min(n, i0 + chunk))
        done[0] += 1
        if done[0] % max(1, len(starts) // 8) == 0:
            say(f"{what}: oracle {done[0]}/{len(starts)} chunks")
        return out

    with threadpool_limits(1):
        with ThreadPoolExecutor(workers) as ex:
            return list(ex.map(run, starts))
