"""Oracle: masked softmax attention, its log-sum-exp merge, streaming form and backward.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  float64 throughout; inputs
are upcast from their stored dtype (bf16 and fp32 values are exact in float64).

Notation (per query row i at global position p_i in document δ_i, head h, and key
row j; q head h reads kv head h // (Hq/Hkv)):
  visible(i, j)  : p_j <= p_i                        (causal on global positions)
                   p_j <= p_i and δ_j == δ_i         (packed, block-diagonal causal)
                   always                            (no mask)
  S_ij = scale · q_i · k_j,  scale = 1/sqrt(d) by default
  LSE_i = log Σ_{visible j} exp S_ij,   O_i = Σ_{visible j} exp(S_ij − LSE_i) v_j
  a row with no visible key has O_i = 0 and LSE_i = −inf.

Sources:
* "Context Parallelism (CP)" page, section 2.1: TileAttention(Q_i, K_j, V_j, M_ij)
  returns the output normalised inside segment j and the per-row LSE of the masked,
  1/sqrt(d)-scaled scores.  Section 2.2: partial states merge by
  L = log Σ exp L_j and O = Σ exp(L_j − L) O_j, associative and commutative.
* "上下文并行：一条序列跨卡，仍算同一个目标" (context-parallel teaching page),
  section 01: the causal rule uses global positions (j <= i), local numbering is
  storage only; section 02: the running-state update m' = max(m, max_B S),
  c = e^{m−m'}, l' = c·l + Σ_B e^{S−m'}, a' = c·a + Σ_B e^{S−m'} V, O = a/l,
  λ = m + log l, and the backward dK_j = Σ_i dS_ij Q_i / sqrt(d),
  dV_j = Σ_i P_ij G_i with contributions from every query rank summed at the owner.
* "Context Parallelism (CP)" page, section 5: packed documents attend causally only
  inside themselves (block-diagonal mask).

Readings where the pages are silent: the diagonal is visible (j <= i); an empty row is
(0, −inf); the grouped-query mapping is contiguous (h // group); the backward's
softmax-Jacobian term uses D_i = Σ_d G_i·O_i (standard softmax derivative).

Pins: tests/test_oracle_attention.py (the 4-token score/softmax table printed on the
"图解 Megatron 的 SP / CP / EP" page, brute-force loops, closed-form special cases,
torch float64 scaled_dot_product_attention and autograd, central finite differences).
"""
from __future__ import annotations

import math

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_CAUSAL_DOC = 2

_BLOCK = 256  # query rows materialised at once


def _f64(x):
    """Upcast a numpy array or a CPU torch tensor (any float dtype) to float64 numpy."""
    if hasattr(x, "detach"):
        import torch
        x = x.detach().to("cpu")
        if x.dtype == torch.bfloat16:
            x = x.to(torch.float32)
        return x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def _i64(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        return x.detach().to("cpu").numpy().astype(np.int64)
    return np.asarray(x, dtype=np.int64)


def visible_mask(q_pos, k_pos, q_doc=None, k_doc=None, mask=MASK_CAUSAL) -> np.ndarray:
    """Boolean [len(q_pos), len(k_pos)]: which (query, key) pairs may attend."""
    q_pos = _i64(q_pos)
    k_pos = _i64(k_pos)
    if mask == MASK_NONE:
        return np.ones((len(q_pos), len(k_pos)), dtype=bool)
    vis = k_pos[None, :] <= q_pos[:, None]
    if mask == MASK_CAUSAL_DOC:
        vis &= _i64(k_doc)[None, :] == _i64(q_doc)[:, None]
    elif mask != MASK_CAUSAL:
        raise ValueError("unknown mask")
    return vis


def _seen_keys(vis):
    """Columns of a visibility block that at least one of its rows can see.

    Restricting a block of query rows to these keys drops only terms that are exactly
    zero (masked probabilities), so every sum keeps its value; it only spares the
    oracle the score rows of keys nobody in the block can see (for a causal share most
    keys, for packed documents nearly all)."""
    return np.flatnonzero(vis.any(axis=0))


def _group(hq, hkv):
    if hq % hkv != 0:
        raise ValueError("hq must be a multiple of hkv")
    return hq // hkv


def attention_fwd(q, k, v, q_pos=None, k_pos=None, q_doc=None, k_doc=None,
                  mask=MASK_CAUSAL, scale=None):
    """Plain masked attention.  q [Tq,Hq,d], k/v [Tk,Hkv,d] -> (O [Tq,Hq,d], LSE [Tq,Hq]).

    Also serves as TileAttention for one (Q block, KV segment) edge: the output is
    normalised over the keys passed in, and LSE is over those keys only."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = _group(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if q_pos is None:
        q_pos = np.arange(tq)
    if k_pos is None:
        k_pos = np.arange(tk)
    o = np.zeros((tq, hq, d))
    lse = np.full((tq, hq), -np.inf)
    if tq == 0 or tk == 0:
        return o, lse
    q_pos, k_pos = _i64(q_pos), _i64(k_pos)
    q_doc, k_doc = _i64(q_doc), _i64(k_doc)
    for r0 in range(0, tq, _BLOCK):
        r1 = min(tq, r0 + _BLOCK)
        vis = visible_mask(q_pos[r0:r1], k_pos,
                           None if q_doc is None else q_doc[r0:r1], k_doc, mask)
        # the keys some row of the block can see (the others add exact zeros)
        cols = _seen_keys(vis)
        vis = vis[:, cols]
        any_vis = vis.any(axis=1)
        for h in range(hq):
            g = h // grp
            s = scale * (q[r0:r1, h, :] @ k[cols, g, :].T)
            s = np.where(vis, s, -np.inf)
            m = np.max(s, axis=1) if len(cols) else np.full(r1 - r0, -np.inf)
            m_safe = np.where(any_vis, m, 0.0)
            p = np.where(vis, np.exp(s - m_safe[:, None]), 0.0)
            l = p.sum(axis=1)
            l_safe = np.where(any_vis, l, 1.0)
            o[r0:r1, h, :] = np.where(any_vis[:, None], (p @ v[cols, g, :]) / l_safe[:, None], 0.0)
            lse[r0:r1, h] = np.where(any_vis, m_safe + np.log(l_safe), -np.inf)
    return o, lse


def merge(parts):
    """Log-sum-exp merge of partial states [(O_j [T,H,d], L_j [T,H]), ...] for the same rows.

    L = log Σ_j exp L_j and O = Σ_j exp(L_j − L) O_j; rows whose parts are all −inf
    stay (0, −inf).  Computed with the row maximum factored out."""
    if len(parts) == 0:
        raise ValueError("need at least one part")
    os_ = [_f64(o) for o, _ in parts]
    ls_ = [_f64(l) for _, l in parts]
    lmax = np.max(np.stack(ls_), axis=0)
    empty = np.isneginf(lmax)
    lmax_safe = np.where(empty, 0.0, lmax)
    tot = np.zeros_like(lmax)
    for l in ls_:
        tot += np.exp(l - lmax_safe)
    lse = np.where(empty, -np.inf, lmax_safe + np.log(np.where(empty, 1.0, tot)))
    lse_safe = np.where(empty, 0.0, lse)
    o = np.zeros_like(os_[0])
    for oj, l in zip(os_, ls_):
        w = np.where(empty, 0.0, np.exp(l - lse_safe))
        o += w[..., None] * oj
    return o, lse


def stream_fwd(q, segments, q_pos=None, q_doc=None, mask=MASK_CAUSAL, scale=None):
    """Streaming (m, l, a) online softmax over KV segments in arrival order.

    ``segments`` is a list of dicts with keys k, v, pos and optionally doc.  For each
    segment B: m' = max(m, max_B S), c = e^{m−m'}, l' = c·l + Σ_B e^{S−m'},
    a' = c·a + Σ_B e^{S−m'} V_B; finally O = a/l and λ = m + log l.  While a row has
    seen no visible key, m stays −inf; the factor c is only formed once m' is finite
    (before that l and a are still zero).  Returns (O, λ) like attention_fwd."""
    q = _f64(q)
    tq, hq, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if q_pos is None:
        q_pos = np.arange(tq)
    q_pos, q_doc = _i64(q_pos), _i64(q_doc)
    m = np.full((tq, hq), -np.inf)
    l = np.zeros((tq, hq))
    a = np.zeros((tq, hq, d))
    for seg in segments:
        k, v = _f64(seg["k"]), _f64(seg["v"])
        if k.shape[0] == 0:
            continue
        grp = _group(hq, k.shape[1])
        vis = visible_mask(q_pos, seg["pos"], q_doc, seg.get("doc"), mask)
        for h in range(hq):
            g = h // grp
            s = scale * (q[:, h, :] @ k[:, g, :].T)
            s = np.where(vis, s, -np.inf)
            m_new = np.maximum(m[:, h], np.max(s, axis=1))
            live = ~np.isneginf(m_new)
            m_new_safe = np.where(live, m_new, 0.0)
            c = np.where(live, np.exp(m[:, h] - m_new_safe), 1.0)
            p = np.where(vis, np.exp(s - m_new_safe[:, None]), 0.0)
            l[:, h] = c * l[:, h] + p.sum(axis=1)
            a[:, h, :] = c[:, None] * a[:, h, :] + p @ v[:, g, :]
            m[:, h] = m_new
    live = l > 0
    o = np.where(live[..., None], a / np.where(live, l, 1.0)[..., None], 0.0)
    lam = np.where(live, m + np.log(np.where(live, l, 1.0)), -np.inf)
    return o, lam


def attention_bwd(q, k, v, g, q_pos=None, k_pos=None, q_doc=None, k_doc=None,
                  mask=MASK_CAUSAL, scale=None, o_saved=None):
    """Gradients of sum(G ∘ O) with O = attention_fwd(q, k, v).  Returns (dQ, dK, dV).

    The forward (O, LSE) is recomputed here in float64; then per visible pair
    P_ij = exp(S_ij − LSE_i), D_i = Σ_d G_i·O_i, dP_ij = G_i·v_j, dS_ij = P_ij(dP_ij − D_i),
    dQ_i = scale Σ_j dS_ij k_j, dK_j = scale Σ_i dS_ij q_i, dV_j = Σ_i P_ij G_i.
    dK/dV of a kv head sum over its query heads.  Rows with no visible key give zero.

    ``o_saved``: the forward output the backward is handed (the teaching page's replay
    uses the saved full-row output, section 01); D_i is then formed from it, e.g. from
    an output stored in bf16, instead of from the recomputed O."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = _group(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if q_pos is None:
        q_pos = np.arange(tq)
    if k_pos is None:
        k_pos = np.arange(tk)
    q_pos, k_pos = _i64(q_pos), _i64(k_pos)
    q_doc, k_doc = _i64(q_doc), _i64(k_doc)
    o, lse = attention_fwd(q, k, v, q_pos, k_pos, q_doc, k_doc, mask, scale)
    if o_saved is not None:
        o = _f64(o_saved)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, tq, _BLOCK):
        r1 = min(tq, r0 + _BLOCK)
        vis = visible_mask(q_pos[r0:r1], k_pos,
                           None if q_doc is None else q_doc[r0:r1], k_doc, mask)
        cols = _seen_keys(vis)
        vis = vis[:, cols]
        for h in range(hq):
            kh = h // grp
            lse_h = lse[r0:r1, h]
            lse_safe = np.where(np.isneginf(lse_h), 0.0, lse_h)
            s = scale * (q[r0:r1, h, :] @ k[cols, kh, :].T)
            p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse_safe[:, None]), 0.0)
            gh = g[r0:r1, h, :]
            dd = np.sum(gh * o[r0:r1, h, :], axis=1)
            dp = gh @ v[cols, kh, :].T
            ds = p * (dp - dd[:, None])
            dq[r0:r1, h, :] += scale * (ds @ k[cols, kh, :])
            dk[cols, kh, :] += scale * (ds.T @ q[r0:r1, h, :])
            dv[cols, kh, :] += p.T @ gh
    return dq, dk, dv


def attention_bwd_keys(q, k, v, g, key_rows, q_pos=None, k_pos=None, q_doc=None, k_doc=None,
                       mask=MASK_CAUSAL, scale=None, o=None, lse=None):
    """dK and dV of sum(G ∘ O) at the chosen key rows only.  Returns ([n, Hkv, d], [n, Hkv, d]).

    The same softmax derivative as ``attention_bwd``, evaluated for the keys
    ``key_rows`` (indices into k / v) against every query row: each query row's
    probabilities are rebuilt from its full-row log-sum-exp over all keys,
    P_ij = exp(S_ij − LSE_i), with D_i = Σ_d G_i·O_i from the full-row output; then
    dK_j = scale Σ_i P_ij (G_i·v_j − D_i) q_i and dV_j = Σ_i P_ij G_i, summed over the
    query heads of each kv head (the per-owner sums of the teaching page, section 01,
    for a subset of the owner's keys).  ``o`` / ``lse`` are the full-row forward
    results of these queries over all of k / v (computed here when not given); a
    given ``o`` is the saved output D is formed from, as for ``attention_bwd``."""
    q, k, v, g = _f64(q), _f64(k), _f64(v), _f64(g)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    grp = _group(hq, hkv)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if q_pos is None:
        q_pos = np.arange(tq)
    if k_pos is None:
        k_pos = np.arange(tk)
    q_pos, k_pos = _i64(q_pos), _i64(k_pos)
    q_doc, k_doc = _i64(q_doc), _i64(k_doc)
    if o is None or lse is None:
        o_f, lse_f = attention_fwd(q, k, v, q_pos, k_pos, q_doc, k_doc, mask, scale)
        o = o_f if o is None else o
        lse = lse_f if lse is None else lse
    o, lse = _f64(o), _f64(lse)
    sel = _i64(key_rows)
    kj, vj = k[sel], v[sel]
    kpos_j = k_pos[sel]
    kdoc_j = None if k_doc is None else k_doc[sel]
    dk = np.zeros((len(sel), hkv, d))
    dv = np.zeros((len(sel), hkv, d))
    if len(sel) == 0 or tq == 0:
        return dk, dv
    for r0 in range(0, tq, _BLOCK):
        r1 = min(tq, r0 + _BLOCK)
        vis = visible_mask(q_pos[r0:r1], kpos_j,
                           None if q_doc is None else q_doc[r0:r1], kdoc_j, mask)
        if not vis.any():
            continue
        for h in range(hq):
            kh = h // grp
            lse_h = lse[r0:r1, h]
            lse_safe = np.where(np.isneginf(lse_h), 0.0, lse_h)
            s = scale * (q[r0:r1, h, :] @ kj[:, kh, :].T)
            p = np.where(vis, np.exp(np.where(vis, s, 0.0) - lse_safe[:, None]), 0.0)
            gh = g[r0:r1, h, :]
            dd = np.sum(gh * o[r0:r1, h, :], axis=1)
            dp = gh @ vj[:, kh, :].T
            ds = p * (dp - dd[:, None])
            dk[:, kh, :] += scale * (ds.T @ q[r0:r1, h, :])
            dv[:, kh, :] += p.T @ gh
    return dk, dv
