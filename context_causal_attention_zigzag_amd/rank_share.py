"""One context-parallel rank's share on one GPU, with the other ranks emulated.

Host-side orchestration only: it decides which buffers form the query blocks and the
KV segments, in which order segments arrive, and which task-graph edges exist; all
arithmetic runs in libcpattn through the C-ABI calls of this package.

* Every owner's K/V shard is produced by the partition kernel (as that owner would
  produce it) and kept as a local buffer standing in for the received segment.
* Ring arrival order for rank r: owners r, r-1, ..., r-cp+1 (mod cp) — the local
  block first, then what arrives from the neighbour, as in the ring tables of the
  "图解 Megatron 的 SP / CP / EP" page (section 5) and the teaching page's owner
  order.  Inside an owner, its chunks keep their storage order (front, then back).
* Edge set of the Q-KV task graph ("Context Parallelism (CP)", section 2.1): an edge
  (query chunk, KV segment) exists when some key position is <= some query position;
  for zigzag shards the library decides this from (S, cp) alone
  (cpattn_zigzag_edge_visible), so empty edges are never launched.  Packed documents
  and striped shards keep every edge (the kernels classify; under the striped split
  every edge holds visible pairs).
* Layouts: "zigzag" (chunk pair), "thd" (packed documents, zigzag inside each) and
  "striped" (rank r holds tokens r, r + cp, ...: the interleaved split of the
  ring-attention page, section 5).
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

from . import (PART_STRIPED, PART_THD, PART_ZIGZAG, MASK_CAUSAL, MASK_CAUSAL_DOC, attn_desc, cpattn_bwd,
               cpattn_bwd_workspace_bytes, cpattn_merge_groups, cpattn_partition, cpattn_stream_fwd,
               cpattn_stream_fwd_workspace_bytes, cpattn_tile_fwd, cpattn_tile_fwd_workspace_bytes,
               cpattn_zigzag_edge_visible, kv_seg, q_block)


def ring_order(cp: int, rank: int):
    return [(rank - i) % cp for i in range(cp)]


@dataclass
class Shard:
    """Rows one owner holds: global indices (positions), doc ids, gathered tensors."""
    owner: int
    idx: torch.Tensor
    doc: torch.Tensor | None
    tensors: list


@dataclass
class RankShare:
    seq: int
    cp: int
    rank: int
    hq: int
    hkv: int
    d: int
    dtype: torch.dtype
    packed: bool
    q: torch.Tensor                      # local queries [S/cp, hq, d]
    q_idx: torch.Tensor                  # their global positions
    q_doc: torch.Tensor | None
    owners: dict = field(default_factory=dict)   # owner -> Shard with [k, v]
    striped: bool = False

    @property
    def mask(self):
        return MASK_CAUSAL_DOC if self.packed else MASK_CAUSAL

    def desc(self, scale: float = 0.0):
        return attn_desc(self.hq, self.hkv, self.d, self.dtype, self.mask, scale)

    # ---- segments ------------------------------------------------------------------
    def segments(self, granularity: str = "owner"):
        """KV segments in ring arrival order: list of (kv_seg, (owner, part), (row0, row1))."""
        out = []
        n = self.seq // self.cp
        for o in ring_order(self.cp, self.rank):
            sh = self.owners[o]
            k, v = sh.tensors
            parts = [(0, n)] if granularity == "owner" else [(0, n // 2), (n // 2, n)]
            for pi, (a, b) in enumerate(parts):
                seg = kv_seg(k[a:b], v[a:b], sh.idx[a:b], None if sh.doc is None else sh.doc[a:b])
                out.append((seg, (o, pi), (a, b)))
        return out

    def q_chunks(self):
        """The local query rows as two chunks (front, back) with their row ranges."""
        n = self.seq // self.cp
        return [(0, n // 2), (n // 2, n)]

    def edges(self, granularity: str = "owner"):
        """Non-empty (query chunk, segment) edges: list of (q rows (a,b), seg, seg index)."""
        segs = self.segments(granularity)
        out = []
        for qi, (a, b) in enumerate(self.q_chunks()):
            for si, (seg, (o, pi), _) in enumerate(segs):
                if not self.packed and not self.striped:
                    kv_part = -1 if granularity == "owner" else pi
                    if not cpattn_zigzag_edge_visible(self.seq, self.cp, self.rank, qi, o, kv_part):
                        continue
                out.append(((a, b), seg, si))
        return out

    # ---- the computations ------------------------------------------------------------
    def stream_fwd(self, granularity="owner", o=None, lse=None, scale=0.0, workspace="auto"):
        n = self.q.shape[0]
        o = torch.empty_like(self.q) if o is None else o
        lse = torch.empty((n, self.hq), dtype=torch.float32, device=self.q.device) if lse is None else lse
        segs = [s for s, _, _ in self.segments(granularity)]
        cpattn_stream_fwd(self.desc(scale), q_block(self.q, self.q_idx, self.q_doc), segs, o, lse,
                          workspace)
        return o, lse

    def stream_workspace(self, granularity="owner", scale=0.0):
        segs = [s for s, _, _ in self.segments(granularity)]
        n = cpattn_stream_fwd_workspace_bytes(self.desc(scale), q_block(self.q, self.q_idx, self.q_doc), segs)
        return torch.empty(n, dtype=torch.uint8, device=self.q.device) if n else None

    def tile_workspace(self, edges, scale=0.0):
        qbs, segs = self._edge_args(edges)
        n = cpattn_tile_fwd_workspace_bytes(self.desc(scale), qbs, segs)
        return torch.empty(n, dtype=torch.uint8, device=self.q.device) if n else None

    def _edge_args(self, edges):
        qbs = []
        for (a, b), _, _ in edges:
            qbs.append(q_block(self.q[a:b], self.q_idx[a:b], None if self.q_doc is None else self.q_doc[a:b]))
        return qbs, [s for _, s, _ in edges]

    def alloc_tile_buffers(self, granularity="owner"):
        edges = self.edges(granularity)
        parts = []
        for (a, b), _, _ in edges:
            parts.append((torch.empty((b - a, self.hq, self.d), dtype=torch.float32, device=self.q.device),
                          torch.empty((b - a, self.hq), dtype=torch.float32, device=self.q.device)))
        return edges, parts

    def tile_fwd(self, edges, parts, scale=0.0, workspace="auto"):
        qbs, segs = self._edge_args(edges)
        cpattn_tile_fwd(self.desc(scale), qbs, segs, [p[0] for p in parts], [p[1] for p in parts], workspace)

    def merge(self, edges, parts, o=None, lse=None):
        n = self.q.shape[0]
        o = torch.empty_like(self.q) if o is None else o
        lse = torch.empty((n, self.hq), dtype=torch.float32, device=self.q.device) if lse is None else lse
        groups = []
        for (a, b) in self.q_chunks():
            mine = [p for e, p in zip(edges, parts) if e[0] == (a, b)]
            if not mine:  # every query chunk sees at least its own diagonal block
                raise ValueError("query chunk without any edge")
            groups.append(([p[0] for p in mine], [p[1] for p in mine], o[a:b], lse[a:b]))
        # every query chunk's merge in one launch
        cpattn_merge_groups(groups)
        return o, lse

    def alloc_bwd_buffers(self, granularity="owner"):
        segs = self.segments(granularity)
        dev = self.q.device
        dq = torch.empty((self.q.shape[0], self.hq, self.d), dtype=torch.float32, device=dev)
        dk = [torch.empty((b - a, self.hkv, self.d), dtype=torch.float32, device=dev) for _, _, (a, b) in segs]
        dv = [torch.empty_like(x) for x in dk]
        segs_ = [s_ for s_, _, _ in segs]
        ws = torch.empty(max(1, cpattn_bwd_workspace_bytes(self.desc(), q_block(self.q, self.q_idx, self.q_doc),
                                                            segs_)), dtype=torch.uint8, device=dev)
        return dq, dk, dv, ws

    def bwd(self, o, lse, g, bufs=None, granularity="owner", scale=0.0):
        dq, dk, dv, ws = self.alloc_bwd_buffers(granularity) if bufs is None else bufs
        segs = [s for s, _, _ in self.segments(granularity)]
        cpattn_bwd(self.desc(scale), q_block(self.q, self.q_idx, self.q_doc), segs, o, lse, g, dq, dk, dv, ws)
        return dq, dk, dv


def partition_shard(mode, total, cp, owner, tensors, cu_host=None, cu_dev=None, with_doc=False):
    """Run the partition kernel for one owner: indices (+doc ids) and gathered tensors."""
    dev = tensors[0].device
    n = total // cp
    idx = torch.empty(n, dtype=torch.int32, device=dev)
    doc = torch.empty(n, dtype=torch.int32, device=dev) if with_doc else None
    outs = [torch.empty((n,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev) for t in tensors]
    cpattn_partition(mode, total, cp, owner, idx, doc, tensors, outs, cu_host, cu_dev)
    return Shard(owner, idx, doc, outs)


def build_rank_share(q_full, k_full, v_full, cp: int, rank: int, cu_seqlens=None,
                     striped: bool = False) -> RankShare:
    """Partition the rank's queries and every owner's K/V on the device (zigzag, packed
    documents when ``cu_seqlens`` is given, or the striped split)."""
    seq, hq, d = q_full.shape
    hkv = k_full.shape[1]
    packed = cu_seqlens is not None
    if packed and striped:
        raise ValueError("the striped split is for one sequence")
    mode = PART_THD if packed else (PART_STRIPED if striped else PART_ZIGZAG)
    cu_dev = None
    if packed:
        cu_dev = torch.as_tensor(list(cu_seqlens), dtype=torch.int32).to(q_full.device)
    qs = partition_shard(mode, seq, cp, rank, [q_full], cu_seqlens, cu_dev, packed)
    rs = RankShare(seq, cp, rank, hq, hkv, d, q_full.dtype, packed, qs.tensors[0], qs.idx, qs.doc,
                   striped=striped)
    for o in range(cp):
        rs.owners[o] = partition_shard(mode, seq, cp, o, [k_full, v_full], cu_seqlens, cu_dev, packed)
    return rs
