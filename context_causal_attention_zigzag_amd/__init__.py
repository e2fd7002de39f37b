"""cpattn: one context-parallel rank's share of causal attention on MI355X (gfx950).

Thin ctypes binding over ``libcpattn.so`` (C ABI declared in ``include/cpattn.h``).
The Python functions carry the C names and only marshal arguments: torch tensors
become device pointers, host tables become ctypes arrays, the current torch stream
becomes the HIP stream.  Every step of the computation runs in the HIP kernels; if
the library is missing this package fails to import.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcpattn.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build the HIP library first "
        "(python -c 'import __graft_entry__ as g; g.build()')")

lib = ctypes.CDLL(LIB_PATH)

# ---- constants (match include/cpattn.h) -------------------------------------------------
OK, ERR_ARG, ERR_ALIGN, ERR_UNSUPPORTED, ERR_HIP, ERR_WORKSPACE = 0, 1, 2, 3, 4, 5
BF16, F32 = 0, 1
MASK_NONE, MASK_CAUSAL, MASK_CAUSAL_DOC = 0, 1, 2
PART_ZIGZAG, PART_THD, PART_STRIPED = 0, 1, 2

_c_i32, _c_i64, _c_f32, _c_vp, _c_sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float,
                                          ctypes.c_void_p, ctypes.c_size_t)


class cpattn_attn_desc(ctypes.Structure):
    _fields_ = [("dtype", _c_i32), ("hq", _c_i32), ("hkv", _c_i32), ("d", _c_i32),
                ("scale", _c_f32), ("mask", _c_i32)]


class cpattn_rope_desc(ctypes.Structure):
    _fields_ = [("rotate_mask", ctypes.c_uint32), ("dtype", _c_i32), ("d", _c_i32),
                ("interleaved", _c_i32), ("base", _c_f32)]


class cpattn_q_block(ctypes.Structure):
    _fields_ = [("q", _c_vp), ("pos", _c_vp), ("doc", _c_vp), ("len", _c_i64)]


class cpattn_kv_seg(ctypes.Structure):
    _fields_ = [("k", _c_vp), ("v", _c_vp), ("pos", _c_vp), ("doc", _c_vp), ("len", _c_i64)]


_P = ctypes.POINTER
lib.cpattn_strerror.argtypes = [_c_i32]
lib.cpattn_strerror.restype = ctypes.c_char_p
lib.cpattn_version.argtypes = []
lib.cpattn_version.restype = _c_i32
lib.cpattn_partition.argtypes = [_c_i32, _c_i64, _c_i32, _c_i32, _P(_c_i32), _c_vp, _c_i32, _c_vp,
                                 _c_vp, _c_i32, _P(_c_vp), _P(_c_vp), _P(_c_i64), _c_vp]
lib.cpattn_partition.restype = _c_i32
lib.cpattn_partition_rope.argtypes = [_c_i32, _c_i64, _c_i32, _c_i32, _P(_c_i32), _c_vp, _c_i32, _c_vp,
                                      _c_vp, _c_i32, _P(_c_vp), _P(_c_vp), _P(_c_i64), _P(cpattn_rope_desc),
                                      _c_vp]
lib.cpattn_partition_rope.restype = _c_i32
lib.cpattn_zigzag_edge_visible.argtypes = [_c_i64, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _P(_c_i32)]
lib.cpattn_zigzag_edge_visible.restype = _c_i32
lib.cpattn_tile_fwd.argtypes = [_P(cpattn_attn_desc), _c_i32, _P(cpattn_q_block), _P(cpattn_kv_seg),
                                _P(_c_vp), _P(_c_vp), _c_vp, _c_sz, _c_vp]
lib.cpattn_tile_fwd.restype = _c_i32
lib.cpattn_tile_fwd_workspace_bytes.argtypes = [_P(cpattn_attn_desc), _c_i32, _P(cpattn_q_block),
                                                _P(cpattn_kv_seg)]
lib.cpattn_tile_fwd_workspace_bytes.restype = _c_sz
lib.cpattn_merge.argtypes = [_c_i32, _P(_c_vp), _P(_c_vp), _c_i64, _c_i32, _c_i32, _c_i32, _c_vp,
                             _c_vp, _c_vp]
lib.cpattn_merge.restype = _c_i32
lib.cpattn_merge_groups.argtypes = [_c_i32, _P(_c_i32), _P(_c_vp), _P(_c_vp), _P(_c_i64), _c_i32, _c_i32, _c_i32,
                                    _P(_c_vp), _P(_c_vp), _c_vp]
lib.cpattn_merge_groups.restype = _c_i32
lib.cpattn_stream_fwd.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32,
                                  _P(cpattn_kv_seg), _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]
lib.cpattn_stream_fwd.restype = _c_i32
lib.cpattn_stream_fwd_workspace_bytes.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32,
                                                  _P(cpattn_kv_seg)]
lib.cpattn_stream_fwd_workspace_bytes.restype = _c_sz
lib.cpattn_bwd.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32, _P(cpattn_kv_seg),
                           _c_vp, _c_vp, _c_vp, _c_vp, _P(_c_vp), _P(_c_vp), _c_vp, _c_sz, _c_vp]
lib.cpattn_bwd.restype = _c_i32
lib.cpattn_bwd_workspace_bytes.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32,
                                           _P(cpattn_kv_seg)]
lib.cpattn_bwd_workspace_bytes.restype = _c_sz
lib.cpattn_bwd_delta.argtypes = [_P(cpattn_attn_desc), _c_i64, _c_vp, _c_vp, _c_vp, _c_vp]
lib.cpattn_bwd_delta.restype = _c_i32
lib.cpattn_bwd_dq.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32, _P(cpattn_kv_seg),
                              _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]
lib.cpattn_bwd_dq.restype = _c_i32
lib.cpattn_bwd_dq_delta.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32, _P(cpattn_kv_seg),
                                    _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_vp, _c_sz, _c_vp]
lib.cpattn_bwd_dq_delta.restype = _c_i32
lib.cpattn_bwd_dq_workspace_bytes.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32,
                                              _P(cpattn_kv_seg)]
lib.cpattn_bwd_dq_workspace_bytes.restype = _c_sz
lib.cpattn_bwd_dkdv.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32, _P(cpattn_kv_seg),
                                _c_vp, _c_vp, _c_vp, _P(_c_vp), _P(_c_vp), _c_vp]
lib.cpattn_bwd_dkdv.restype = _c_i32

lib.cpattn_bwd_noalloc.argtypes = [_P(cpattn_attn_desc), _P(cpattn_q_block), _c_i32, _P(cpattn_kv_seg),
                                   _c_vp, _c_vp, _c_vp, _c_vp, _P(_c_vp), _P(_c_vp), _c_vp]
lib.cpattn_bwd_noalloc.restype = _c_i32

EXPORTED = ("cpattn_strerror", "cpattn_version", "cpattn_partition", "cpattn_partition_rope",
            "cpattn_zigzag_edge_visible", "cpattn_tile_fwd",
            "cpattn_tile_fwd_workspace_bytes", "cpattn_merge", "cpattn_merge_groups", "cpattn_stream_fwd",
            "cpattn_stream_fwd_workspace_bytes", "cpattn_bwd", "cpattn_bwd_workspace_bytes",
            "cpattn_bwd_delta", "cpattn_bwd_dq", "cpattn_bwd_dq_delta", "cpattn_bwd_dq_workspace_bytes", "cpattn_bwd_dkdv",
            "cpattn_bwd_noalloc")


class CpattnError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: status {status}: {cpattn_strerror(status)}")


def cpattn_strerror(status: int) -> str:
    return lib.cpattn_strerror(status).decode()


def _check(status: int, where: str):
    if status != OK:
        raise CpattnError(status, where)


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to cpattn must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


_DT = {torch.bfloat16: BF16, torch.float32: F32}


def attn_desc(hq: int, hkv: int, d: int, dtype=torch.bfloat16, mask: int = MASK_CAUSAL,
              scale: float = 0.0) -> cpattn_attn_desc:
    return cpattn_attn_desc(_DT[dtype] if not isinstance(dtype, int) else dtype, hq, hkv, d,
                            float(scale), mask)


def q_block(q, pos, doc=None) -> cpattn_q_block:
    n = 0 if q is None else q.shape[0]
    return cpattn_q_block(_ptr(q) if n else None, _ptr(pos) if n else None,
                          _ptr(doc) if (n and doc is not None) else None, n)


def kv_seg(k, v, pos, doc=None) -> cpattn_kv_seg:
    n = 0 if k is None else k.shape[0]
    return cpattn_kv_seg(_ptr(k) if n else None, _ptr(v) if n else None,
                         _ptr(pos) if n else None, _ptr(doc) if (n and doc is not None) else None, n)


def _vp_array(ptrs):
    return (_c_vp * max(1, len(ptrs)))(*ptrs)


# ---- the five calls ---------------------------------------------------------------------
def rope_desc(rotate=(0, 1), dtype=torch.bfloat16, d: int = 128, interleaved: bool = False,
              base: float = 10000.0) -> cpattn_rope_desc:
    """Rotary options of cpattn_partition_rope: ``rotate`` lists the gathered tensors to rotate."""
    mask = 0
    for g in rotate:
        mask |= 1 << g
    return cpattn_rope_desc(mask, _DT[dtype] if not isinstance(dtype, int) else dtype, d, int(interleaved),
                            float(base))


def cpattn_partition(mode: int, total: int, cp_size: int, cp_rank: int, idx_out, doc_out=None,
                     src=(), dst=(), cu_seqlens_host=None, cu_seqlens_dev=None, stream=None, rope=None):
    """Rows of rank ``cp_rank`` (zigzag, per-document or striped) into ``idx_out`` (+ ``doc_out``),
    and ``dst[g][i] = src[g][idx_out[i]]`` for every tensor pair; with ``rope`` (a
    cpattn_rope_desc) the selected tensors are rotated on the way (cpattn_partition_rope)."""
    if len(src) != len(dst):
        raise ValueError("src and dst must pair up")
    row_bytes = [math.prod(s.shape[1:]) * s.element_size() for s in src]
    cu_host = None
    n_docs = 0
    if mode == PART_THD:
        vals = [int(x) for x in cu_seqlens_host]
        n_docs = len(vals) - 1
        cu_host = (_c_i32 * len(vals))(*vals)
    args = (mode, total, cp_size, cp_rank, cu_host, _ptr(cu_seqlens_dev), n_docs, _ptr(idx_out), _ptr(doc_out),
            len(src), _vp_array([_ptr(s) for s in src]), _vp_array([_ptr(d) for d in dst]),
            (_c_i64 * max(1, len(src)))(*row_bytes))
    if rope is None:
        _check(lib.cpattn_partition(*args, _stream(stream)), "cpattn_partition")
    else:
        _check(lib.cpattn_partition_rope(*args, ctypes.byref(rope), _stream(stream)), "cpattn_partition_rope")


def cpattn_zigzag_edge_visible(seq_len: int, cp_size: int, q_rank: int, q_part: int, kv_owner: int,
                               kv_part: int) -> bool:
    """Whether the (query block, KV segment) edge of a zigzag share has visible pairs
    (part: 0 front chunk, 1 back chunk, -1 both)."""
    out = _c_i32(0)
    _check(lib.cpattn_zigzag_edge_visible(seq_len, cp_size, q_rank, q_part, kv_owner, kv_part, ctypes.byref(out)),
           "cpattn_zigzag_edge_visible")
    return bool(out.value)


def _workspace(nbytes, like, stream=None):
    """A device buffer of ``nbytes`` (None for 0), allocated through torch on the stream
    the kernels will run on: when the caller drops it, torch's caching allocator only
    hands the block to later work of that same stream, which runs after the kernels."""
    if nbytes == 0:
        return None
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=like.device)
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream, device=like.device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=like.device)


def _ws_args(ws):
    if ws is None:
        return None, 0
    return _ptr(ws), ws.numel() * ws.element_size()


def cpattn_tile_fwd_workspace_bytes(desc: cpattn_attn_desc, q_blocks, segs) -> int:
    n = len(q_blocks)
    qa = (cpattn_q_block * max(1, n))(*q_blocks)
    sa = (cpattn_kv_seg * max(1, n))(*segs)
    return int(lib.cpattn_tile_fwd_workspace_bytes(ctypes.byref(desc), n, qa, sa))


def cpattn_tile_fwd(desc: cpattn_attn_desc, q_blocks, segs, o_parts, lse_parts, workspace="auto",
                    stream=None):
    """TileAttention for every (q_blocks[e], segs[e]) edge into (o_parts[e], lse_parts[e]).

    ``workspace``: a uint8 device tensor, None (no KV split), or "auto" (sized with
    cpattn_tile_fwd_workspace_bytes and allocated here)."""
    n = len(q_blocks)
    if not (len(segs) == len(o_parts) == len(lse_parts) == n):
        raise ValueError("one q block, segment, O and LSE buffer per edge")
    if isinstance(workspace, str):
        workspace = (_workspace(cpattn_tile_fwd_workspace_bytes(desc, q_blocks, segs), o_parts[0], stream)
                     if n else None)
    qa = (cpattn_q_block * max(1, n))(*q_blocks)
    sa = (cpattn_kv_seg * max(1, n))(*segs)
    wp, wb = _ws_args(workspace)
    st = lib.cpattn_tile_fwd(ctypes.byref(desc), n, qa, sa, _vp_array([_ptr(o) for o in o_parts]),
                             _vp_array([_ptr(x) for x in lse_parts]), wp, wb, _stream(stream))
    _check(st, "cpattn_tile_fwd")


def cpattn_merge(o_parts, lse_parts, o_out, lse_out, stream=None):
    """Log-sum-exp merge of fp32 partial states into (o_out, lse_out)."""
    n = len(o_parts)
    rows, hq, d = o_out.shape
    out_dtype = _DT[o_out.dtype]
    st = lib.cpattn_merge(n, _vp_array([_ptr(o) for o in o_parts]),
                          _vp_array([_ptr(x) for x in lse_parts]), rows, hq, d, out_dtype,
                          _ptr(o_out), _ptr(lse_out), _stream(stream))
    _check(st, "cpattn_merge")


def cpattn_merge_groups(groups, stream=None):
    """Several log-sum-exp merges in one launch: ``groups`` is a list of
    (o_parts, lse_parts, o_out, lse_out), each as for cpattn_merge; all outputs share
    one dtype, head count and head dim."""
    n = len(groups)
    if n == 0:
        return
    _, hq, d = groups[0][2].shape
    out_dtype = _DT[groups[0][2].dtype]
    n_parts = (_c_i32 * n)(*[len(g[0]) for g in groups])
    rows = (_c_i64 * n)(*[g[2].shape[0] for g in groups])
    o_parts = _vp_array([_ptr(o) for g in groups for o in g[0]])
    lse_parts = _vp_array([_ptr(x) for g in groups for x in g[1]])
    st = lib.cpattn_merge_groups(n, n_parts, o_parts, lse_parts, rows, hq, d, out_dtype,
                                 _vp_array([_ptr(g[2]) for g in groups]), _vp_array([_ptr(g[3]) for g in groups]),
                                 _stream(stream))
    _check(st, "cpattn_merge_groups")


def cpattn_stream_fwd_workspace_bytes(desc: cpattn_attn_desc, q: cpattn_q_block, segs) -> int:
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    return int(lib.cpattn_stream_fwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(q), len(segs), sa))


def cpattn_stream_fwd(desc: cpattn_attn_desc, q: cpattn_q_block, segs, o_out, lse_out, workspace="auto",
                      stream=None):
    """Streaming online-softmax attention of ``q`` over ``segs`` in arrival order.

    ``workspace`` as for cpattn_tile_fwd (cpattn_stream_fwd_workspace_bytes)."""
    if isinstance(workspace, str):
        workspace = (_workspace(cpattn_stream_fwd_workspace_bytes(desc, q, segs), o_out, stream)
                     if o_out is not None else None)
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    wp, wb = _ws_args(workspace)
    st = lib.cpattn_stream_fwd(ctypes.byref(desc), ctypes.byref(q), len(segs), sa, _ptr(o_out),
                               _ptr(lse_out), wp, wb, _stream(stream))
    _check(st, "cpattn_stream_fwd")


def cpattn_bwd_workspace_bytes(desc: cpattn_attn_desc, q: cpattn_q_block, segs) -> int:
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    return int(lib.cpattn_bwd_workspace_bytes(ctypes.byref(desc), ctypes.byref(q), len(segs), sa))


def cpattn_bwd(desc: cpattn_attn_desc, q: cpattn_q_block, segs, o, lse, dout, dq, dk, dv,
               workspace, stream=None):
    """LSE-replay backward: dQ for the local rows, per-segment summed dK/dV."""
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    st = lib.cpattn_bwd(ctypes.byref(desc), ctypes.byref(q), len(segs), sa, _ptr(o), _ptr(lse),
                        _ptr(dout), _ptr(dq), _vp_array([_ptr(x) for x in dk]),
                        _vp_array([_ptr(x) for x in dv]), _ptr(workspace),
                        0 if workspace is None else workspace.numel() * workspace.element_size(),
                        _stream(stream))
    _check(st, "cpattn_bwd")


def cpattn_bwd_delta(desc: cpattn_attn_desc, o, dout, delta, stream=None):
    """D = rowsum(dout * o) per (row, head) into fp32 ``delta`` [rows, hq]."""
    rows = 0 if o is None else o.shape[0]
    st = lib.cpattn_bwd_delta(ctypes.byref(desc), rows, _ptr(o) if rows else None,
                              _ptr(dout) if rows else None, _ptr(delta) if rows else None, _stream(stream))
    _check(st, "cpattn_bwd_delta")


def cpattn_bwd_dq_workspace_bytes(desc: cpattn_attn_desc, q: cpattn_q_block, segs) -> int:
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    return int(lib.cpattn_bwd_dq_workspace_bytes(ctypes.byref(desc), ctypes.byref(q), len(segs), sa))


def cpattn_bwd_dq(desc: cpattn_attn_desc, q: cpattn_q_block, segs, lse, delta, dout, dq, workspace=None,
                  stream=None):
    """dQ pass of the backward (``workspace``: uint8 device tensor or None = unsplit)."""
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    wp, wb = _ws_args(workspace)
    st = lib.cpattn_bwd_dq(ctypes.byref(desc), ctypes.byref(q), len(segs), sa, _ptr(lse), _ptr(delta),
                           _ptr(dout), _ptr(dq), wp, wb, _stream(stream))
    _check(st, "cpattn_bwd_dq")


def cpattn_bwd_dq_delta(desc: cpattn_attn_desc, q: cpattn_q_block, segs, o, lse, dout, delta, dq,
                        workspace=None, stream=None):
    """dQ pass that also forms the per-row values D from O and dO and stores them in ``delta``."""
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    wp, wb = _ws_args(workspace)
    st = lib.cpattn_bwd_dq_delta(ctypes.byref(desc), ctypes.byref(q), len(segs), sa, _ptr(o), _ptr(lse),
                                 _ptr(dout), _ptr(delta), _ptr(dq), wp, wb, _stream(stream))
    _check(st, "cpattn_bwd_dq_delta")


def cpattn_bwd_dkdv(desc: cpattn_attn_desc, q: cpattn_q_block, segs, lse, delta, dout, dk, dv,
                    stream=None):
    """dK/dV pass of the backward: per-segment sums over all local rows."""
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    st = lib.cpattn_bwd_dkdv(ctypes.byref(desc), ctypes.byref(q), len(segs), sa, _ptr(lse), _ptr(delta),
                             _ptr(dout), _vp_array([_ptr(x) for x in dk]), _vp_array([_ptr(x) for x in dv]),
                             _stream(stream))
    _check(st, "cpattn_bwd_dkdv")


def cpattn_bwd_noalloc(desc: cpattn_attn_desc, q: cpattn_q_block, segs, o, lse, dout, dq, dk, dv, stream=None):
    """cpattn_bwd with the library's per-device scratch array as its workspace."""
    sa = (cpattn_kv_seg * max(1, len(segs)))(*segs)
    st = lib.cpattn_bwd_noalloc(ctypes.byref(desc), ctypes.byref(q), len(segs), sa, _ptr(o), _ptr(lse),
                                _ptr(dout), _ptr(dq), _vp_array([_ptr(x) for x in dk]),
                                _vp_array([_ptr(x) for x in dv]), _stream(stream))
    _check(st, "cpattn_bwd_noalloc")
