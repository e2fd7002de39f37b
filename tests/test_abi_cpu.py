"""The C-ABI library loads, exports what include/cpattn.h declares, and rejects bad
arguments on the host before touching a GPU (CPU only: no compute call is made)."""
import ctypes
import os
import re
import subprocess

import pytest
import torch

import context_causal_attention_zigzag_amd as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cpattn_\w+)\s*\(", text)))


def test_header_declares_the_five_calls():
    names = declared_functions()
    for n in ("cpattn_partition", "cpattn_tile_fwd", "cpattn_merge", "cpattn_stream_fwd", "cpattn_bwd"):
        assert n in names


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", C.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (cpattn_\w+)", out))
    for n in declared_functions():
        assert n in exported, n
        assert hasattr(C.lib, n)
    assert set(C.EXPORTED) == set(declared_functions())


def test_strerror_names_every_status():
    for st in range(6):
        assert C.cpattn_strerror(st) and "unknown" not in C.cpattn_strerror(st)
    assert "unknown" in C.cpattn_strerror(99)


FAKE = 0x100000  # never dereferenced: every call below fails validation first


def part(mode, total, cp, rank, cu=None, n_gather=0, row_bytes=(16,)):
    cu_arr = (ctypes.c_int32 * len(cu))(*cu) if cu else None
    n_docs = len(cu) - 1 if cu else 0
    ptrs = (ctypes.c_void_p * 1)(FAKE)
    rb = (ctypes.c_int64 * 1)(*row_bytes)
    return C.lib.cpattn_partition(mode, total, cp, rank, cu_arr, FAKE if cu else None, n_docs, FAKE, None,
                                  n_gather, ptrs, ptrs, rb, None)


def test_partition_validation():
    assert part(C.PART_ZIGZAG, 100, 4, 0) == C.ERR_ALIGN          # 100 % 8
    assert part(C.PART_ZIGZAG, 64, 4, 4) == C.ERR_ARG             # rank out of range
    assert part(C.PART_ZIGZAG, 64, 0, 0) == C.ERR_ARG
    assert part(C.PART_ZIGZAG, -8, 2, 0) == C.ERR_ARG
    assert part(7, 64, 2, 0) == C.ERR_ARG
    assert part(C.PART_THD, 64, 2, 0, cu=[0, 32, 60]) == C.ERR_ALIGN   # does not end at total
    assert part(C.PART_THD, 64, 2, 0, cu=[0, 30, 64]) == C.ERR_ALIGN   # 30 % 4
    assert part(C.PART_THD, 64, 2, 0, cu=[0, 40, 32, 64]) == C.ERR_ALIGN  # not monotone
    assert part(C.PART_THD, 64, 2, 0, cu=[1, 32, 64]) == C.ERR_ALIGN
    assert part(C.PART_ZIGZAG, 64, 2, 0, n_gather=1, row_bytes=(24,)) == C.ERR_ALIGN
    assert part(C.PART_ZIGZAG, 64, 2, 0, n_gather=1, row_bytes=(0,)) == C.ERR_ARG
    assert part(C.PART_ZIGZAG, 64, 2, 0, n_gather=9) == C.ERR_ARG


def desc(**kw):
    base = dict(dtype=C.BF16, hq=8, hkv=8, d=128, scale=0.0, mask=C.MASK_CAUSAL)
    base.update(kw)
    return C.cpattn_attn_desc(**base)


def qb(n=64, q=FAKE):
    return C.cpattn_q_block(q, FAKE, None, n)


def sg(n=64):
    return C.cpattn_kv_seg(FAKE, FAKE, FAKE, None, n)


def stream_call(d, q=None, segs=None):
    q = q or qb()
    segs = segs if segs is not None else [sg()]
    arr = (C.cpattn_kv_seg * max(1, len(segs)))(*segs)
    return C.lib.cpattn_stream_fwd(ctypes.byref(d), ctypes.byref(q), len(segs), arr, FAKE, FAKE, None, 0, None)


def test_attention_validation():
    assert stream_call(desc(d=96)) == C.ERR_UNSUPPORTED
    assert stream_call(desc(hq=6, hkv=4)) == C.ERR_UNSUPPORTED
    assert stream_call(desc(mask=5)) == C.ERR_UNSUPPORTED
    assert stream_call(desc(dtype=7)) == C.ERR_UNSUPPORTED
    assert stream_call(desc(hkv=0)) == C.ERR_ARG
    assert stream_call(desc(scale=float("nan"))) == C.ERR_ARG
    assert stream_call(desc(), segs=[]) == C.ERR_ARG
    assert stream_call(desc(), segs=[sg()] * 33) == C.ERR_WORKSPACE   # two groups of segments need a workspace
    assert stream_call(desc(), segs=[sg()] * 2049) == C.ERR_ARG
    assert stream_call(desc(), q=qb(q=FAKE + 8)) == C.ERR_ALIGN
    assert stream_call(desc(), q=C.cpattn_q_block(FAKE, None, None, 64)) == C.ERR_ARG
    assert stream_call(desc(mask=C.MASK_CAUSAL_DOC)) == C.ERR_ARG     # doc ids required
    assert stream_call(desc(), segs=[C.cpattn_kv_seg(FAKE, FAKE, FAKE, None, -1)]) == C.ERR_ARG


def test_tile_and_merge_validation():
    d = desc(d=64)
    q = (C.cpattn_q_block * 1)(qb())
    s = (C.cpattn_kv_seg * 1)(sg())
    nul = (ctypes.c_void_p * 1)(None)
    assert C.lib.cpattn_tile_fwd(ctypes.byref(d), 1, q, s, nul, nul, None, 0, None) == C.ERR_ARG
    assert C.lib.cpattn_tile_fwd(ctypes.byref(d), -1, q, s, nul, nul, None, 0, None) == C.ERR_ARG
    assert C.lib.cpattn_tile_fwd(ctypes.byref(d), 0, q, s, nul, nul, None, 0, None) == C.OK   # no-op
    p1 = (ctypes.c_void_p * 1)(FAKE)
    assert C.lib.cpattn_tile_fwd(ctypes.byref(d), 1, q, s, p1, p1, FAKE + 16, 1 << 20, None) == C.ERR_ALIGN
    p = (ctypes.c_void_p * 1)(FAKE)
    assert C.lib.cpattn_merge(0, p, p, 10, 8, 128, C.BF16, FAKE, FAKE, None) == C.ERR_ARG
    assert C.lib.cpattn_merge(65, p, p, 10, 8, 128, C.BF16, FAKE, FAKE, None) == C.ERR_ARG
    assert C.lib.cpattn_merge(1, p, p, 10, 8, 6, C.BF16, FAKE, FAKE, None) == C.ERR_UNSUPPORTED
    assert C.lib.cpattn_merge(1, p, p, 10, 8, 128, 9, FAKE, FAKE, None) == C.ERR_UNSUPPORTED
    assert C.lib.cpattn_merge(1, p, p, 0, 8, 128, C.BF16, FAKE, FAKE, None) == C.OK   # no-op


def test_merge_groups_validation():
    def call(n_groups, n_parts, rows, d=128, dtype=C.BF16, parts=None, outs=None, hq=8):
        np_ = (ctypes.c_int32 * max(1, len(n_parts)))(*n_parts)
        rw = (ctypes.c_int64 * max(1, len(rows)))(*rows)
        total = sum(max(0, x) for x in n_parts)
        pp = parts if parts is not None else (ctypes.c_void_p * max(1, total))(*([FAKE] * max(1, total)))
        oo = outs if outs is not None else (ctypes.c_void_p * max(1, len(rows)))(*([FAKE] * max(1, len(rows))))
        return C.lib.cpattn_merge_groups(n_groups, np_, pp, pp, rw, hq, d, dtype, oo, oo, None)
    assert call(-1, [], []) == C.ERR_ARG
    assert call(0, [], []) == C.OK                                   # no-op
    assert call(2, [1, 2], [10, 10], hq=0) == C.ERR_ARG
    assert call(2, [1, 2], [10, 10], d=6) == C.ERR_UNSUPPORTED
    assert call(2, [1, 2], [10, 10], dtype=9) == C.ERR_UNSUPPORTED
    assert call(2, [1, 0], [10, 10]) == C.ERR_ARG                    # a group without parts
    assert call(2, [1, 65], [10, 10]) == C.ERR_ARG
    assert call(2, [1, 2], [10, -1]) == C.ERR_ARG
    nul = (ctypes.c_void_p * 3)(FAKE, None, FAKE)
    assert call(2, [1, 2], [10, 10], parts=nul) == C.ERR_ARG         # a null part
    mis = (ctypes.c_void_p * 3)(FAKE, FAKE + 8, FAKE)
    assert call(2, [1, 2], [10, 10], parts=mis) == C.ERR_ALIGN       # a misaligned part
    out_nul = (ctypes.c_void_p * 2)(FAKE, None)
    assert call(2, [1, 2], [10, 10], outs=out_nul) == C.ERR_ARG      # a null output
    assert call(2, [1, 2], [0, 0], outs=out_nul) == C.OK             # groups of 0 rows: outputs not read


def test_forward_workspace_plan():
    # a small share (2048 rows x 8 heads, 4 segments of 2048 keys) cannot fill 256 CUs
    # with query tiles alone: a split is planned; a large one (64 query tiles x 64 heads) not
    d = desc()
    q = qb(2048)
    segs = (C.cpattn_kv_seg * 4)(*[sg(2048)] * 4)
    small = C.lib.cpattn_stream_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(q), 4, segs)
    assert small > 0 and small % 256 == 0
    big = desc(hq=64, hkv=64)
    qbig = qb(8192)
    assert C.lib.cpattn_stream_fwd_workspace_bytes(ctypes.byref(big), ctypes.byref(qbig), 4, segs) == 0
    assert C.lib.cpattn_stream_fwd_workspace_bytes(ctypes.byref(desc(dtype=C.F32)), ctypes.byref(q), 4, segs) == 0
    # edges of 64 KV tiles are split; edges of 32 tiles or fewer never are
    qa = (C.cpattn_q_block * 2)(qb(1024), qb(1024))
    sa = (C.cpattn_kv_seg * 2)(sg(4096), sg(4096))
    assert C.lib.cpattn_tile_fwd_workspace_bytes(ctypes.byref(d), 2, qa, sa) > 0
    sa32 = (C.cpattn_kv_seg * 2)(sg(2048), sg(2048))
    assert C.lib.cpattn_tile_fwd_workspace_bytes(ctypes.byref(d), 2, qa, sa32) == 0


def test_bwd_validation_and_workspace():
    d = desc()
    s1 = (C.cpattn_kv_seg * 1)(sg(64))
    q3 = qb(3)
    assert C.lib.cpattn_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(q3), 1, s1) == 256
    big = desc(hq=64, hkv=64)
    q8k = qb(8192)
    assert C.lib.cpattn_bwd_workspace_bytes(ctypes.byref(big), ctypes.byref(q8k), 1, s1) == 8192 * 64 * 4
    segs4 = (C.cpattn_kv_seg * 4)(*[sg(2048)] * 4)
    q = qb(2048)
    assert C.lib.cpattn_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(q), 4, segs4) > 2048 * 8 * 4
    assert C.lib.cpattn_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(qb(-1)), 4, segs4) == 0
    s = (C.cpattn_kv_seg * 1)(sg())
    p = (ctypes.c_void_p * 1)(FAKE)
    f32 = desc(dtype=C.F32)
    assert C.lib.cpattn_bwd(ctypes.byref(f32), ctypes.byref(q), 1, s, FAKE, FAKE, FAKE, FAKE, p, p,
                            FAKE, 1 << 20, None) == C.ERR_UNSUPPORTED
    assert C.lib.cpattn_bwd(ctypes.byref(d), ctypes.byref(q), 1, s, FAKE, FAKE, FAKE, FAKE, p, p,
                            FAKE, 100, None) == C.ERR_WORKSPACE
    assert C.lib.cpattn_bwd(ctypes.byref(d), ctypes.byref(qb((1 << 30) + 1)), 1, s, FAKE, FAKE, FAKE, FAKE, p, p,
                            FAKE, 1 << 30, None) == C.ERR_ARG
    assert C.lib.cpattn_bwd(ctypes.byref(d), ctypes.byref(q), 1, s, FAKE, FAKE, FAKE, FAKE, p, p,
                            None, 1 << 20, None) == C.ERR_WORKSPACE
    nul = (ctypes.c_void_p * 1)(None)
    assert C.lib.cpattn_bwd(ctypes.byref(d), ctypes.byref(q), 1, s, FAKE, FAKE, FAKE, FAKE, nul, p,
                            FAKE, 1 << 20, None) == C.ERR_ARG


def test_bwd_pass_calls_validation():
    d = desc()
    f32 = desc(dtype=C.F32)
    lib = C.lib
    # delta: dtype, size, pointers, alignment; zero rows is a no-op that touches nothing
    assert lib.cpattn_bwd_delta(ctypes.byref(f32), 64, FAKE, FAKE, FAKE, None) == C.ERR_UNSUPPORTED
    assert lib.cpattn_bwd_delta(ctypes.byref(d), -1, FAKE, FAKE, FAKE, None) == C.ERR_ARG
    assert lib.cpattn_bwd_delta(ctypes.byref(d), 0, None, None, None, None) == C.OK
    assert lib.cpattn_bwd_delta(ctypes.byref(d), 64, FAKE, None, FAKE, None) == C.ERR_ARG
    assert lib.cpattn_bwd_delta(ctypes.byref(d), 64, FAKE + 8, FAKE, FAKE, None) == C.ERR_ALIGN
    s4 = (C.cpattn_kv_seg * 4)(*[sg(2048)] * 4)
    q = qb(2048)
    # dQ workspace = the combined call's workspace minus the delta rows
    full = lib.cpattn_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(q), 4, s4)
    assert lib.cpattn_bwd_dq_workspace_bytes(ctypes.byref(d), ctypes.byref(q), 4, s4) == full - 2048 * 8 * 4
    assert lib.cpattn_bwd_dq_workspace_bytes(ctypes.byref(f32), ctypes.byref(q), 4, s4) == 0
    assert lib.cpattn_bwd_dq_workspace_bytes(ctypes.byref(d), ctypes.byref(q), 0, s4) == 0
    # dQ: missing per-row inputs, output, alignment
    assert lib.cpattn_bwd_dq(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE, None, FAKE, FAKE, None, 0,
                             None) == C.ERR_ARG
    assert lib.cpattn_bwd_dq(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE, None, None, 0,
                             None) == C.ERR_ARG
    assert lib.cpattn_bwd_dq(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE + 4, FAKE, None, 0,
                             None) == C.ERR_ALIGN
    assert lib.cpattn_bwd_dq(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE, FAKE, FAKE + 16,
                             1 << 20, None) == C.ERR_ALIGN
    assert lib.cpattn_bwd_dq(ctypes.byref(d), ctypes.byref(qb(0)), 4, s4, None, None, None, None, None, 0,
                             None) == C.OK
    # dQ forming delta: the forward output is needed (and aligned) when there are rows
    assert lib.cpattn_bwd_dq_delta(ctypes.byref(d), ctypes.byref(q), 4, s4, None, FAKE, FAKE, FAKE, FAKE, None, 0,
                                   None) == C.ERR_ARG
    assert lib.cpattn_bwd_dq_delta(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE + 8, FAKE, FAKE, FAKE, FAKE, None,
                                   0, None) == C.ERR_ALIGN
    assert lib.cpattn_bwd_dq_delta(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE, None, FAKE, None, 0,
                                   None) == C.ERR_ARG
    assert lib.cpattn_bwd_dq_delta(ctypes.byref(f32), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE, FAKE, FAKE, None,
                                   0, None) == C.ERR_UNSUPPORTED
    assert lib.cpattn_bwd_dq_delta(ctypes.byref(d), ctypes.byref(qb(0)), 4, s4, None, None, None, None, None, None,
                                   0, None) == C.OK
    # dK/dV: row limit, output tables, alignment
    p = (ctypes.c_void_p * 4)(*[FAKE] * 4)
    nul = (ctypes.c_void_p * 4)(FAKE, FAKE, None, FAKE)
    odd = (ctypes.c_void_p * 4)(FAKE, FAKE + 4, FAKE, FAKE)
    assert lib.cpattn_bwd_dkdv(ctypes.byref(d), ctypes.byref(qb((1 << 30) + 1)), 4, s4, FAKE, FAKE, FAKE, p, p,
                               None) == C.ERR_ARG
    assert lib.cpattn_bwd_dkdv(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE, None, p,
                               None) == C.ERR_ARG
    assert lib.cpattn_bwd_dkdv(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE, p, nul,
                               None) == C.ERR_ARG
    assert lib.cpattn_bwd_dkdv(ctypes.byref(d), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE, odd, p,
                               None) == C.ERR_ALIGN
    assert lib.cpattn_bwd_dkdv(ctypes.byref(f32), ctypes.byref(q), 4, s4, FAKE, FAKE, FAKE, p, p,
                               None) == C.ERR_UNSUPPORTED


def test_bwd_noalloc_validation():
    # rejected on the host before any device work: dtype, sizes, and per-row values
    # larger than the library's scratch array (CPATTN_NOALLOC_SCRATCH_BYTES, 64 MiB)
    d, f32 = desc(), desc(dtype=C.F32)
    s = (C.cpattn_kv_seg * 1)(sg())
    p = (ctypes.c_void_p * 1)(FAKE)
    rest = (FAKE, FAKE, FAKE, FAKE, p, p, None)
    assert C.lib.cpattn_bwd_noalloc(ctypes.byref(f32), ctypes.byref(qb(64)), 1, s, *rest) == C.ERR_UNSUPPORTED
    assert C.lib.cpattn_bwd_noalloc(ctypes.byref(d), ctypes.byref(qb(-1)), 1, s, *rest) == C.ERR_ARG
    wide = desc(hq=64, hkv=8)
    rows = (64 << 20) // (64 * 4) + 1
    assert C.lib.cpattn_bwd_noalloc(ctypes.byref(wide), ctypes.byref(qb(rows)), 1, s, *rest) == C.ERR_WORKSPACE
    text = open(HEADER).read()
    assert "#define CPATTN_NOALLOC_SCRATCH_BYTES (64u << 20)" in text


def test_striped_and_rope_partition_validation():
    # striped: the length must divide by cp (not 2cp); checked before any launch
    assert part(C.PART_STRIPED, 10, 4, 0) == C.ERR_ALIGN
    assert part(3, 64, 2, 0) == C.ERR_ARG
    ptrs = (ctypes.c_void_p * 2)(FAKE, FAKE)

    def rope_call(rope, row_bytes=(256, 256), n_gather=2):
        rb = (ctypes.c_int64 * 2)(*row_bytes)
        return C.lib.cpattn_partition_rope(C.PART_ZIGZAG, 64, 2, 0, None, None, 0, FAKE, None, n_gather, ptrs, ptrs,
                                           rb, None if rope is None else ctypes.byref(rope), None)

    ok = dict(rotate=(0, 1), dtype=torch.bfloat16, d=128)
    assert rope_call(None) == C.ERR_ARG
    assert rope_call(C.rope_desc(rotate=(0, 2))) == C.ERR_ARG            # tensor 2 is not gathered
    r = C.rope_desc(**ok)
    r.dtype = 7
    assert rope_call(r) == C.ERR_UNSUPPORTED
    assert rope_call(C.rope_desc(rotate=(0,), d=8)) == C.ERR_UNSUPPORTED
    assert rope_call(C.rope_desc(rotate=(0,), d=72)) == C.ERR_UNSUPPORTED
    assert rope_call(C.rope_desc(rotate=(0,), d=272)) == C.ERR_UNSUPPORTED
    r = C.rope_desc(**ok)
    r.interleaved = 2
    assert rope_call(r) == C.ERR_ARG
    assert rope_call(C.rope_desc(base=-1.0, **ok)) == C.ERR_ARG
    assert rope_call(C.rope_desc(base=float("inf"), **ok)) == C.ERR_ARG
    assert rope_call(C.rope_desc(**ok), row_bytes=(256, 48)) == C.ERR_ALIGN  # 48 B: not a whole head
    # the plain partition's own checks come first
    rb = (ctypes.c_int64 * 1)(256)
    assert C.lib.cpattn_partition_rope(C.PART_ZIGZAG, 100, 4, 0, None, None, 0, FAKE, None, 1, ptrs, ptrs, rb,
                                       ctypes.byref(C.rope_desc(**ok)), None) == C.ERR_ALIGN


def test_segment_and_row_limits():
    # up to 2048 segments per call (groups of 32 per launch); more is refused
    d = desc()
    q = qb(1024)
    segs = (C.cpattn_kv_seg * 2049)(*[sg(64)] * 2049)
    p = (ctypes.c_void_p * 2049)(*[FAKE] * 2049)
    assert C.lib.cpattn_stream_fwd(ctypes.byref(d), ctypes.byref(q), 2049, segs, FAKE, FAKE, None, 0,
                                   None) == C.ERR_ARG
    assert C.lib.cpattn_bwd_dkdv(ctypes.byref(d), ctypes.byref(q), 2049, segs, FAKE, FAKE, FAKE, p, p,
                                 None) == C.ERR_ARG
    # more than 32 segments: the streaming form needs one fp32 partial state per group of 32
    want = 2 * (((1024 * 8 * 128 * 4 + 255) // 256) * 256 + ((1024 * 8 * 4 + 255) // 256) * 256)
    assert C.lib.cpattn_stream_fwd_workspace_bytes(ctypes.byref(d), ctypes.byref(q), 40, segs) == want
    assert C.lib.cpattn_stream_fwd(ctypes.byref(d), ctypes.byref(q), 40, segs, FAKE, FAKE, None, 0,
                                   None) == C.ERR_WORKSPACE
    assert C.lib.cpattn_stream_fwd(ctypes.byref(d), ctypes.byref(q), 40, segs, FAKE, FAKE, FAKE, want - 256,
                                   None) == C.ERR_WORKSPACE
    # and the dQ pass of a grouped list runs unsplit: no split workspace is planned
    assert C.lib.cpattn_bwd_dq_workspace_bytes(ctypes.byref(d), ctypes.byref(q), 40, segs) == 0
    assert C.lib.cpattn_bwd_workspace_bytes(ctypes.byref(d), ctypes.byref(q), 40, segs) == 1024 * 8 * 4


def test_zigzag_edge_visible_matches_the_causal_mask():
    # brute force over the oracle's zigzag rows: an edge has work iff some key position
    # of the segment is <= some query position of the block
    import numpy as np
    import oracle

    out = ctypes.c_int32(-1)
    checked = 0
    for seq, cp in [(16, 1), (32, 2), (64, 4), (96, 3), (128, 8), (8192, 4)]:
        chunk = seq // (2 * cp)
        for r in range(cp):
            rows_q = oracle.zigzag_indices(seq, cp, r)
            for o in range(cp):
                rows_k = oracle.zigzag_indices(seq, cp, o)
                for qp in (-1, 0, 1):
                    q = rows_q if qp < 0 else rows_q[qp * chunk:(qp + 1) * chunk]
                    for kp in (-1, 0, 1):
                        k = rows_k if kp < 0 else rows_k[kp * chunk:(kp + 1) * chunk]
                        want = bool(np.any(k[:, None] <= q[None, :]))
                        assert C.lib.cpattn_zigzag_edge_visible(seq, cp, r, qp, o, kp, ctypes.byref(out)) == C.OK
                        assert bool(out.value) == want, (seq, cp, r, qp, o, kp)
                        assert C.cpattn_zigzag_edge_visible(seq, cp, r, qp, o, kp) == want
                        checked += 1
    assert checked == 990
    # the diagonal edge always has work; rank 0's front chunk sees no later owner
    assert C.cpattn_zigzag_edge_visible(8192, 4, 2, 0, 2, 0)
    assert not C.cpattn_zigzag_edge_visible(8192, 4, 0, 0, 1, -1)
    bad = [(0, 2, 0, 0, 0, 0), (64, 0, 0, 0, 0, 0), (64, 2, 2, 0, 0, 0), (64, 2, 0, 2, 0, 0),
           (64, 2, 0, 0, -1, 0), (64, 2, 0, 0, 0, -2)]
    for args in bad:
        assert C.lib.cpattn_zigzag_edge_visible(*args, ctypes.byref(out)) == C.ERR_ARG, args
    assert C.lib.cpattn_zigzag_edge_visible(66, 2, 0, 0, 0, 0, ctypes.byref(out)) == C.ERR_ALIGN
    assert C.lib.cpattn_zigzag_edge_visible(64, 2, 0, 0, 0, 0, None) == C.ERR_ARG
