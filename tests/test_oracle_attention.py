"""Pins for the attention oracle (CPU only).

What fixes the answers:
* the 4-token score matrix and its softmax rows printed on the "图解 Megatron 的 SP /
  CP / EP" page (section 2.2, step ③), within the 3-decimal print;
* brute force with explicit Python loops on tiny inputs;
* closed forms: a single visible key gives O = v_j and LSE = s_ij; all-zero queries
  give the mean of the visible values and LSE = log(#visible); no visible key gives
  (0, -inf);
* torch's float64 scaled_dot_product_attention (causal, grouped-query) and float64
  autograd as an independent library implementation;
* central finite differences of sum(G∘O);
* the identities the pages state: merged shards equal full attention ("Context
  Parallelism (CP)" page, section 2.2), merge order does not matter, the streaming
  update equals the plain result (ring-attention page, section 2; teaching page,
  section 02), and K/V gradients summed at their owners equal the full gradients
  (teaching page, section 01).
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as A
from oracle import partition as P

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rnd(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- printed example
def _four_token():
    g = json.load(open(os.path.join(GOLDEN, "four_token_softmax.json")))
    s = np.array(g["scores"])[:, None, :]          # q rows = score rows, [4,1,4]
    eye = np.eye(4)[:, None, :]                    # k = v = I4 -> q.k = score, O = P
    return g, s, eye


def test_four_token_softmax_rows():
    g, s, eye = _four_token()
    o, lse = A.attention_fwd(s, eye, eye, mask=A.MASK_NONE, scale=1.0)
    want = np.array(g["softmax"])
    assert np.max(np.abs(o[:, 0, :] - want)) <= g["tolerance"]
    assert np.allclose(o[:, 0, :].sum(axis=1), 1.0, atol=1e-14)
    sc = np.array(g["scores"])
    assert np.allclose(lse[:, 0], np.log(np.exp(sc).sum(axis=1)), atol=1e-14)


def test_four_token_split_into_two_segments_and_merged():
    g, s, eye = _four_token()
    parts = []
    for cols in ([0, 1], [2, 3]):
        parts.append(A.attention_fwd(s, eye[cols], eye[cols], mask=A.MASK_NONE, scale=1.0))
    o, lse = A.merge(parts)
    o_full, lse_full = A.attention_fwd(s, eye, eye, mask=A.MASK_NONE, scale=1.0)
    assert np.max(np.abs(o - o_full)) < 1e-14 and np.max(np.abs(lse - lse_full)) < 1e-14
    assert np.max(np.abs(o[:, 0, :] - np.array(g["softmax"]))) <= g["tolerance"]


# ---------------------------------------------------------------- brute force
def brute(q, k, v, qp, kp, qd, kd, mask, scale):
    tq, hq, d = q.shape
    grp = hq // k.shape[1]
    o = np.zeros(q.shape)
    lse = np.full((tq, hq), -math.inf)
    for i in range(tq):
        for h in range(hq):
            g = h // grp
            vis = []
            for j in range(k.shape[0]):
                ok = True
                if mask >= A.MASK_CAUSAL:
                    ok = kp[j] <= qp[i]
                if mask == A.MASK_CAUSAL_DOC:
                    ok = ok and kd[j] == qd[i]
                if ok:
                    vis.append(j)
            if not vis:
                continue
            sc = [scale * sum(q[i, h, t] * k[j, g, t] for t in range(d)) for j in vis]
            den = sum(math.exp(x) for x in sc)
            lse[i, h] = math.log(den)
            for t in range(d):
                o[i, h, t] = sum(math.exp(x) * v[j, g, t] for x, j in zip(sc, vis)) / den
    return o, lse


@pytest.mark.parametrize("mask", [A.MASK_NONE, A.MASK_CAUSAL, A.MASK_CAUSAL_DOC])
@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2)])
def test_brute_force_tiny(mask, hq, hkv):
    rng = np.random.default_rng(7 + mask + hq)
    tq, tk, d = 7, 11, 3
    q, k, v = rng.standard_normal((tq, hq, d)), rng.standard_normal((tk, hkv, d)), rng.standard_normal((tk, hkv, d))
    qp = rng.permutation(16)[:tq]          # arbitrary, unsorted global positions
    kp = rng.permutation(16)[:tk]
    qd = rng.integers(0, 2, tq)
    kd = rng.integers(0, 2, tk)
    scale = 0.37
    o, lse = A.attention_fwd(q, k, v, qp, kp, qd, kd, mask, scale)
    ob, lb = brute(q, k, v, qp, kp, qd, kd, mask, scale)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = ~np.isneginf(lb)
    assert np.max(np.abs(lse[fin] - lb[fin])) < 1e-12
    assert np.max(np.abs(o - ob)) < 1e-12


# ---------------------------------------------------------------- closed forms
def test_single_visible_key_and_empty_rows():
    rng = np.random.default_rng(3)
    q, k, v = rng.standard_normal((3, 1, 4)), rng.standard_normal((3, 1, 4)), rng.standard_normal((3, 1, 4))
    qp = np.array([0, 5, -1])      # row 0 sees key 0 only; row 2 sees nothing
    kp = np.array([0, 6, 7])
    o, lse = A.attention_fwd(q, k, v, qp, kp, scale=0.5)
    assert np.allclose(o[0, 0], v[0, 0], atol=1e-15)
    assert abs(lse[0, 0] - 0.5 * q[0, 0] @ k[0, 0]) < 1e-15
    assert np.all(o[2] == 0) and np.isneginf(lse[2, 0])
    assert np.all(o[1] == o[1]) and not np.any(np.isnan(o))


def test_constant_scores_give_mean_of_visible_values():
    rng = np.random.default_rng(4)
    t = 9
    q = np.zeros((t, 2, 5))
    k, v = rng.standard_normal((t, 2, 5)), rng.standard_normal((t, 2, 5))
    o, lse = A.attention_fwd(q, k, v)
    for i in range(t):
        assert np.allclose(o[i], v[: i + 1].mean(axis=0), atol=1e-14)
        assert np.allclose(lse[i], math.log(i + 1), atol=1e-14)


def test_empty_inputs():
    o, lse = A.attention_fwd(np.zeros((0, 2, 4)), np.zeros((5, 2, 4)), np.zeros((5, 2, 4)))
    assert o.shape == (0, 2, 4) and lse.shape == (0, 2)
    o, lse = A.attention_fwd(np.ones((3, 2, 4)), np.zeros((0, 2, 4)), np.zeros((0, 2, 4)))
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# ---------------------------------------------------------------- library cross-check
@pytest.mark.parametrize("hq,hkv", [(4, 4), (8, 2)])
def test_against_torch_sdpa_float64(hq, hkv):
    t, d = 300, 16                     # 300 rows: more than one 256-row block
    q, k, v = rnd((t, hq, d), 1), rnd((t, hkv, d), 2), rnd((t, hkv, d), 3)
    o, lse = A.attention_fwd(q, k, v)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None]
    tk = torch.from_numpy(k).permute(1, 0, 2)[None]
    tv = torch.from_numpy(v).permute(1, 0, 2)[None]
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True,
                                                           enable_gqa=(hq != hkv))
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(o - ref)) < 1e-12
    # LSE from torch.logsumexp of masked scores
    grp = hq // hkv
    kk = torch.from_numpy(k).repeat_interleave(grp, dim=1)
    s = torch.einsum("thd,shd->hts", torch.from_numpy(q), kk) / math.sqrt(d)
    s = s.masked_fill(torch.triu(torch.ones(t, t, dtype=torch.bool), 1), -math.inf)
    lse_ref = torch.logsumexp(s, dim=-1).T.numpy()
    assert np.max(np.abs(lse - lse_ref)) < 1e-12


def test_backward_against_torch_autograd_float64():
    t, hq, hkv, d = 70, 4, 2, 8
    q, k, v, g = rnd((t, hq, d), 11), rnd((t, hkv, d), 12), rnd((t, hkv, d), 13), rnd((t, hq, d), 14)
    dq, dk, dv = A.attention_bwd(q, k, v, g)
    tq = torch.from_numpy(q).permute(1, 0, 2)[None].requires_grad_()
    tk = torch.from_numpy(k).permute(1, 0, 2)[None].requires_grad_()
    tv = torch.from_numpy(v).permute(1, 0, 2)[None].requires_grad_()
    out = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True, enable_gqa=True)
    (out * torch.from_numpy(g).permute(1, 0, 2)[None]).sum().backward()
    assert np.max(np.abs(dq - tq.grad[0].permute(1, 0, 2).numpy())) < 1e-12
    assert np.max(np.abs(dk - tk.grad[0].permute(1, 0, 2).numpy())) < 1e-12
    assert np.max(np.abs(dv - tv.grad[0].permute(1, 0, 2).numpy())) < 1e-12


@pytest.mark.parametrize("mask", [A.MASK_CAUSAL, A.MASK_CAUSAL_DOC])
def test_backward_finite_differences(mask):
    rng = np.random.default_rng(21)
    tq, tk, hq, hkv, d = 5, 6, 2, 1, 3
    q, k, v, g = (rng.standard_normal(s) for s in [(tq, hq, d), (tk, hkv, d), (tk, hkv, d), (tq, hq, d)])
    qp, kp = np.array([1, 3, 4, 6, -2]), np.array([0, 1, 2, 3, 5, 6])
    qd, kd = np.array([0, 0, 1, 1, 1]), np.array([0, 0, 0, 1, 1, 1])
    args = dict(q_pos=qp, k_pos=kp, q_doc=qd, k_doc=kd, mask=mask, scale=0.6)
    dq, dk, dv = A.attention_bwd(q, k, v, g, **args)

    def loss(qq, kk, vv):
        return float(np.sum(A.attention_fwd(qq, kk, vv, **args)[0] * g))

    eps = 1e-6
    for x, dx, which in ((q, dq, 0), (k, dk, 1), (v, dv, 2)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            a = [q, k, v]
            a[which] = xp
            lp = loss(*a)
            a[which] = xm
            lm = loss(*a)
            num[idx] = (lp - lm) / (2 * eps)
        assert np.max(np.abs(num - dx)) <= 1e-6 * max(1.0, np.max(np.abs(dx)))
    assert np.all(dq[4] == 0)   # row at position -2 sees nothing: zero gradient


# ---------------------------------------------------------------- pages' identities
def _chunk_rows(seq, cp, c):
    ch = seq // (2 * cp)
    return np.arange(c * ch, (c + 1) * ch)


@pytest.mark.parametrize("seq,cp,hq,hkv", [(64, 2, 2, 2), (96, 3, 4, 2)])
def test_zigzag_shards_merged_equal_full(seq, cp, hq, hkv):
    d = 8
    q, k, v = rnd((seq, hq, d), 31), rnd((seq, hkv, d), 32), rnd((seq, hkv, d), 33)
    o_full, lse_full = A.attention_fwd(q, k, v)
    for r in range(cp):
        rows = P.zigzag_indices(seq, cp, r)
        parts = []
        for c in range(2 * cp):          # every KV chunk, including fully masked ones
            kr = _chunk_rows(seq, cp, c)
            parts.append(A.attention_fwd(q[rows], k[kr], v[kr], rows, kr))
        o, lse = A.merge(parts)
        assert np.max(np.abs(o - o_full[rows])) < 1e-13
        assert np.max(np.abs(lse - lse_full[rows])) < 1e-13


def test_merge_order_and_grouping_do_not_matter():
    rng = np.random.default_rng(5)
    t, h, d = 6, 2, 3
    parts = [(rng.standard_normal((t, h, d)), rng.standard_normal((t, h)) * 3) for _ in range(4)]
    parts[2][1][0, :] = -np.inf       # a fully masked row in one part
    ident = (np.zeros((t, h, d)), np.full((t, h), -np.inf))
    ref = A.merge(parts)
    for perm in itertools.permutations(range(4)):
        o, l = A.merge([parts[i] for i in perm])
        assert np.max(np.abs(o - ref[0])) < 1e-13 and np.max(np.abs(l - ref[1])) < 1e-13
    tree = A.merge([A.merge(parts[:2]), A.merge([parts[2], ident, parts[3]])])
    assert np.max(np.abs(tree[0] - ref[0])) < 1e-13 and np.max(np.abs(tree[1] - ref[1])) < 1e-13
    o, l = A.merge([ident, ident])
    assert np.all(o == 0) and np.all(np.isneginf(l))


def test_merge_is_not_an_average():
    # block-wise softmax then equal-weight averaging is wrong (teaching page, section 02)
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((4, 1, 3)), rng.standard_normal((6, 1, 3)), rng.standard_normal((6, 1, 3))
    a = A.attention_fwd(q, k[:2], v[:2], mask=A.MASK_NONE)
    b = A.attention_fwd(q, k[2:], v[2:], mask=A.MASK_NONE)
    full = A.attention_fwd(q, k, v, mask=A.MASK_NONE)
    assert np.max(np.abs(A.merge([a, b])[0] - full[0])) < 1e-14
    assert np.max(np.abs(0.5 * (a[0] + b[0]) - full[0])) > 1e-3


def test_stream_equals_plain_two_owners_unequal_segments():
    # five positions, 2-D Q/K/V, owners {0,1} and {2,3,4} (teaching page, sections 01 and 05)
    rng = np.random.default_rng(8)
    q, k, v = rng.standard_normal((5, 1, 2)), rng.standard_normal((5, 1, 2)), rng.standard_normal((5, 1, 2))
    own = [np.array([0, 1]), np.array([2, 3, 4])]
    full = A.attention_fwd(q, k, v)
    for order in ([0, 1], [1, 0]):
        segs = [dict(k=k[own[o]], v=v[own[o]], pos=own[o]) for o in order]
        o, lam = A.stream_fwd(q, segs)
        assert np.max(np.abs(o - full[0])) < 1e-14 and np.max(np.abs(lam - full[1])) < 1e-14
    # per-owner gradient sums with the global-mean upstream G/5 equal the full gradient
    g = rng.standard_normal((5, 1, 2)) / 5
    dq_f, dk_f, dv_f = A.attention_bwd(q, k, v, g)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for qr in own:                     # each query owner replays every KV owner
        for kr in own:
            # partial backward restricted to one KV owner, using the full-row LSE/output
            o_all, lse_all = A.attention_fwd(q[qr], k, v, qr, np.arange(5))
            s = (q[qr, 0] @ k[kr, 0].T) / math.sqrt(2)
            vis = kr[None, :] <= qr[:, None]
            p = np.where(vis, np.exp(s - lse_all[:, 0:1]), 0.0)
            dd = np.sum(g[qr, 0] * o_all[:, 0], axis=1)
            ds = p * (g[qr, 0] @ v[kr, 0].T - dd[:, None])
            dk[kr, 0] += ds.T @ q[qr, 0] / math.sqrt(2)
            dv[kr, 0] += p.T @ g[qr, 0]
    assert np.max(np.abs(dk - dk_f)) < 1e-14 and np.max(np.abs(dv - dv_f)) < 1e-14


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_stream_equals_plain_random_orders(seed):
    rng = np.random.default_rng(seed)
    t, hq, hkv, d = 40, 4, 2, 5
    q, k, v = rng.standard_normal((t, hq, d)), rng.standard_normal((t, hkv, d)), rng.standard_normal((t, hkv, d))
    qrows = np.sort(rng.permutation(t)[:17])
    cuts = np.sort(rng.choice(np.arange(1, t), 4, replace=False))
    segs_rows = np.split(rng.permutation(t), cuts)     # unequal, unsorted segments
    full = A.attention_fwd(q[qrows], k, v, qrows, np.arange(t))
    order = rng.permutation(len(segs_rows))
    segs = [dict(k=k[segs_rows[i]], v=v[segs_rows[i]], pos=segs_rows[i]) for i in order]
    o, lam = A.stream_fwd(q[qrows], segs, qrows)
    assert np.max(np.abs(o - full[0])) < 1e-13 and np.max(np.abs(lam - full[1])) < 1e-13


def test_owner_sums_over_emulated_ranks_equal_full_gradients():
    seq, cp, hq, hkv, d = 48, 3, 2, 1, 4
    q, k, v, g = rnd((seq, hq, d), 41), rnd((seq, hkv, d), 42), rnd((seq, hkv, d), 43), rnd((seq, hq, d), 44)
    dq_f, dk_f, dv_f = A.attention_bwd(q, k, v, g)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r in range(cp):
        rows = P.zigzag_indices(seq, cp, r)
        dq_r, dk_r, dv_r = A.attention_bwd(q[rows], k, v, g[rows], rows, np.arange(seq))
        assert np.max(np.abs(dq_r - dq_f[rows])) < 1e-13
        dk += dk_r
        dv += dv_r
    assert np.max(np.abs(dk - dk_f)) < 1e-13 and np.max(np.abs(dv - dv_f)) < 1e-13


def test_packed_documents_do_not_interact():
    rng = np.random.default_rng(9)
    lens = [8, 16, 8]
    cu = np.concatenate([[0], np.cumsum(lens)])
    t, h, d = cu[-1], 2, 4
    q, k, v = rng.standard_normal((t, h, d)), rng.standard_normal((t, h, d)), rng.standard_normal((t, h, d))
    doc = np.searchsorted(cu, np.arange(t), side="right") - 1
    o, lse = A.attention_fwd(q, k, v, np.arange(t), np.arange(t), doc, doc, A.MASK_CAUSAL_DOC)
    for a, b in zip(cu[:-1], cu[1:]):
        oo, ll = A.attention_fwd(q[a:b], k[a:b], v[a:b])
        assert np.max(np.abs(o[a:b] - oo)) < 1e-14 and np.max(np.abs(lse[a:b] - ll)) < 1e-14


# ---------------------------------------------------------------- dK/dV at chosen keys
def _torch_share_grads(q, k, v, g, qpos, kpos, qdoc=None, kdoc=None, scale=None):
    """dK, dV of sum(G∘O) for queries at positions qpos against every key, by float64
    autograd over an explicitly masked softmax (an independent formulation)."""
    tq, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    scale = 1.0 / math.sqrt(d) if scale is None else scale
    tk_ = torch.from_numpy(k).requires_grad_()
    tv_ = torch.from_numpy(v).requires_grad_()
    vis = torch.from_numpy(kpos)[None, :] <= torch.from_numpy(qpos)[:, None]
    if qdoc is not None:
        vis &= torch.from_numpy(kdoc)[None, :] == torch.from_numpy(qdoc)[:, None]
    loss = 0.0
    for h in range(hq):
        s = scale * torch.from_numpy(q[:, h, :]) @ tk_[:, h // grp, :].T
        s = s.masked_fill(~vis, -math.inf)
        p = torch.softmax(s, dim=1).nan_to_num(0.0)
        loss = loss + (p @ tv_[:, h // grp, :] * torch.from_numpy(g[:, h, :])).sum()
    loss.backward()
    return tk_.grad.numpy(), tv_.grad.numpy()


@pytest.mark.parametrize("hq,hkv", [(1, 1), (4, 2)])
def test_bwd_keys_against_autograd_for_a_rank_share(hq, hkv):
    seq, cp, r, d = 48, 3, 1, 8
    q, k, v = rnd((seq, hq, d), 51), rnd((seq, hkv, d), 52), rnd((seq, hkv, d), 53)
    rows = P.zigzag_indices(seq, cp, r)
    g = rnd((len(rows), hq, d), 54)
    keys = np.array([0, 5, 8, 15, 16, 23, 31, 40, 47])   # the last ones no local query sees
    dk, dv = A.attention_bwd_keys(q[rows], k, v, g, keys, rows, np.arange(seq))
    dk_t, dv_t = _torch_share_grads(q[rows], k, v, g, rows, np.arange(seq))
    assert np.max(np.abs(dk - dk_t[keys])) < 1e-12
    assert np.max(np.abs(dv - dv_t[keys])) < 1e-12
    # rank 1 of cp=3 holds chunks 1 and 4 (positions 8..15 and 32..39): keys after 39
    # are seen by nobody, and their gradients are exactly zero
    assert np.all(dk[-2:] == 0) and np.all(dv[-2:] == 0)
    assert np.max(np.abs(dk[:3])) > 0.1


def test_bwd_keys_document_mask_against_autograd():
    rng = np.random.default_rng(61)
    cu = [0, 16, 40, 48]
    t, hq, hkv, d = 48, 2, 2, 4
    q, k, v = (rng.standard_normal((t, h, d)) for h in (hq, hkv, hkv))
    rows = P.thd_indices(cu, 2, 0)
    qdoc = P.thd_doc_ids(cu, rows)
    kdoc = P.thd_doc_ids(cu, np.arange(t))
    g = rng.standard_normal((len(rows), hq, d))
    keys = np.array([0, 3, 15, 16, 20, 39, 40, 47])
    args = dict(q_doc=qdoc, k_doc=kdoc, mask=A.MASK_CAUSAL_DOC)
    dk, dv = A.attention_bwd_keys(q[rows], k, v, g, keys, rows, np.arange(t), **args)
    dk_t, dv_t = _torch_share_grads(q[rows], k, v, g, rows, np.arange(t), qdoc, kdoc)
    assert np.max(np.abs(dk - dk_t[keys])) < 1e-12
    assert np.max(np.abs(dv - dv_t[keys])) < 1e-12


def test_bwd_keys_with_given_forward_matches_full_backward_rows():
    seq, hq, hkv, d = 40, 2, 1, 4
    q, k, v, g = rnd((seq, hq, d), 71), rnd((seq, hkv, d), 72), rnd((seq, hkv, d), 73), rnd((seq, hq, d), 74)
    o, lse = A.attention_fwd(q, k, v)
    keys = np.arange(0, seq, 3)
    dk1, dv1 = A.attention_bwd_keys(q, k, v, g, keys, o=o, lse=lse)
    dk2, dv2 = A.attention_bwd_keys(q, k, v, g, keys)
    _, dk_f, dv_f = A.attention_bwd(q, k, v, g)
    assert np.array_equal(dk1, dk2) and np.array_equal(dv1, dv2)
    assert np.max(np.abs(dk1 - dk_f[keys])) < 1e-13 and np.max(np.abs(dv1 - dv_f[keys])) < 1e-13


def test_bwd_saved_output_only_enters_through_d():
    # D_i = G_i . O_i is the only place the saved output enters: with the exact output
    # nothing changes; with another output dQ and dK move, dV (= P^T G) does not
    seq, hq, hkv, d = 30, 2, 1, 4
    q, k, v, g = rnd((seq, hq, d), 81), rnd((seq, hkv, d), 82), rnd((seq, hkv, d), 83), rnd((seq, hq, d), 84)
    o, _ = A.attention_fwd(q, k, v)
    base = A.attention_bwd(q, k, v, g)
    same = A.attention_bwd(q, k, v, g, o_saved=o)
    assert all(np.array_equal(a, b) for a, b in zip(base, same))
    o2 = o + 1e-3 * rnd(o.shape, 85)
    dq2, dk2, dv2 = A.attention_bwd(q, k, v, g, o_saved=o2)
    assert np.array_equal(dv2, base[2])
    assert np.max(np.abs(dq2 - base[0])) > 1e-6 and np.max(np.abs(dk2 - base[1])) > 1e-6
    # and it matches the chosen-keys form given the same saved output
    keys = np.arange(0, seq, 4)
    dk3, dv3 = A.attention_bwd_keys(q, k, v, g, keys, o=o2)
    assert np.max(np.abs(dk3 - dk2[keys])) < 1e-13 and np.max(np.abs(dv3 - dv2[keys])) < 1e-13
