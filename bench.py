"""Benchmark: one context-parallel rank's share of causal attention on one MI355X.

Workload (default): S=8192 tokens, cp=4 zigzag, rank 0, H=8 (MHA), d=128, bf16 — the
rank holds chunks 0 and 7 (2048 query rows); the four owners' K/V shards (2048 rows
each) are resident in HBM as the segments the ring would deliver, in arrival order.

One step = the whole hot path for that share:
  partition (this rank's Q, K, V rows)  -> tile forward over the task-graph edges
  -> LSE merge per query chunk -> streaming forward over the 4 segments
  -> LSE-replay backward (dQ, per-owner dK/dV) with upstream G.
Useful FLOPs count visible (query, key) pairs only: S(S+1)/(2cp) per head for every
zigzag rank; forward 4*d per pair per head (QK^T and PV), backward 10*d (five
contractions).  value = useful FLOPs of the step (two forwards + one backward) / time.
The backward runs as its two calls (dQ forming the per-row values D, then dK/dV) so
each is timed on its own.

Prints one JSON line (rank 0).  For the 8K share every rank, on the zigzag and on the
striped split, is then timed in interleaved rounds after a common warm-up (median of
three rounds per share), reported as ``per_rank_tflops`` (min and mean over the ranks)
and ``striped_vs_zigzag``.
``--workload s128k`` runs the 128K share instead; ``--workload thd64k`` a packed stream
of 65536 tokens in documents of lognormal lengths, split per document (zigzag inside
each document, cp=4, rank 1 by default),
with the document mask; its visible pairs are counted per row from the partition's
position and document outputs.
``--copy-mib N`` only runs a plain device copy of N MiB (``--steps`` times): the
known-size reference that calibrates the FETCH_SIZE / WRITE_SIZE counters.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)
CSRC = os.path.join(ROOT, "context_causal_attention_zigzag_amd", "csrc")
# kernel -> (source files it is built from, counter summary under profiles/)
# timed call -> the kernel it launches (rocprofv3 names it with its template arguments)
KERNEL_OF = {"partition": "partition_kernel", "merge": "merge_kernel<true>",
             "bwd_dkdv": "bwd_dkdv_kernel<{d}, ...>", "tile_fwd": "fwd_bf16_kernel<{d}, ...>",
             "stream_fwd": "fwd_bf16_kernel<{d}, ...>", "bwd_dq": "bwd_dq_kernel<{d}, ...>"}
TRAFFIC = {"bwd_dkdv": (("bwd.hip", "kv_stream.h", "common.h"), "bwd_dkdv_kernel_{w}_traffic.txt")}


class TimingEvent:
    """A HIP event for timing only, created with hipEventDisableSystemFence.

    A default event record ends in a system-scope fence that writes back and
    invalidates the caches; that costs GPU time between the kernels it separates and
    slows the kernel after it (cold caches).  Without the fence the event still waits
    for the work before it on the stream and takes its timestamp there, which is all
    a timing needs (the loop is read only after a device synchronisation).  Recorded
    on torch's current stream, the stream the library launches on."""
    _hip = None
    DISABLE_SYSTEM_FENCE = 0x20000000  # hip_runtime_api.h

    def __init__(self):
        import ctypes
        import torch
        if TimingEvent._hip is None:
            # the HIP runtime torch has loaded (same soname, so the same instance)
            hip = ctypes.CDLL("libamdhip64.so.7")
            hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
            TimingEvent._hip = hip
        self._torch = torch
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        self._check(self._hip.hipEventCreateWithFlags(ctypes.byref(self.ev), self.DISABLE_SYSTEM_FENCE),
                    "hipEventCreateWithFlags")

    @staticmethod
    def _check(rc, what):
        if rc != 0:
            raise RuntimeError(f"{what} failed with HIP error {rc}")

    def record(self):
        s = self._torch.cuda.current_stream().cuda_stream
        self._check(self._hip.hipEventRecord(self.ev, self._ct.c_void_p(s)), "hipEventRecord")

    def elapsed_time(self, end) -> float:
        ms = self._ct.c_float()
        self._check(self._hip.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev), "hipEventElapsedTime")
        return ms.value

    def __del__(self):
        if self._hip is not None and self.ev:
            self._hip.hipEventDestroy(self.ev)


def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(kernel, workload):
    """HBM bytes per launch from the committed counter summary, or None when there is
    none or the kernel's sources changed since the counters were taken."""
    if kernel not in TRAFFIC:
        return None
    files, name = TRAFFIC[kernel]
    path = os.path.join(ROOT, "profiles", name.format(w=workload))
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if ":" in line and not line.startswith("#"):
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    if kv.get("source_sha256") != source_hash(files):
        return None
    return int(float(kv["traffic_bytes_per_launch"]))


def copy_calibration(mib, reps):
    import torch
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": reps}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="s8k", choices=["s8k", "s128k", "thd64k"])
    ap.add_argument("--rank", type=int, default=None)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-mib", type=int, default=0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: the other ranks' KV segments are "
                                   "emulated as local buffers; --gpus above 1 is not supported"}))
        sys.exit(2)
    if args.copy_mib:
        copy_calibration(args.copy_mib, args.steps)
        return

    import numpy as np
    import torch

    import workloads
    from context_causal_attention_zigzag_amd.rank_share import (build_rank_share, partition_shard,
                                                                 ring_order)
    import context_causal_attention_zigzag_amd as C

    dev = "cuda"
    w = workloads.WORKLOADS[args.workload]
    r = w.ranks[0] if args.rank is None else args.rank
    q, k, v = workloads.full_qkv(w)
    gq, gk, gv = q.to(dev), k.to(dev), v.to(dev)
    gran = w.kv_granularity
    cu = workloads.cu_seqlens_from_lengths(workloads.thd_lengths(w.seed)) if w.packed else None
    cu_dev = torch.as_tensor(cu, dtype=torch.int32, device=dev) if w.packed else None
    part_mode = C.PART_THD if w.packed else C.PART_ZIGZAG
    n_local = w.seq // w.cp
    names = ["partition", "tile_fwd", "merge", "stream_fwd", "bwd_dq", "bwd_dkdv"]

    def share_steps(rank, striped=False):
        """Buffers of one rank's share and the function running one step of it."""
        rs = build_rank_share(gq, gk, gv, w.cp, rank, cu, striped=striped)
        mode = C.PART_STRIPED if striped else part_mode
        g = workloads.randn((n_local, w.hq, w.d), 5, "bf16", 3).to(dev)
        edges, parts = rs.alloc_tile_buffers(gran)
        o_t = torch.empty_like(rs.q)
        l_t = torch.empty((n_local, w.hq), dtype=torch.float32, device=dev)
        o_s = torch.empty_like(rs.q)
        l_s = torch.empty_like(l_t)
        dq, dk, dv, _ = rs.alloc_bwd_buffers(gran)
        desc = rs.desc()
        qblk = C.q_block(rs.q, rs.q_idx, rs.q_doc)
        bsegs = [s_ for s_, _, _ in rs.segments(gran)]
        delta = torch.empty((n_local, w.hq), dtype=torch.float32, device=dev)
        ws_dq = torch.empty(max(1, C.cpattn_bwd_dq_workspace_bytes(desc, qblk, bsegs)), dtype=torch.uint8,
                            device=dev)
        ws_tile = rs.tile_workspace(edges)
        ws_stream = rs.stream_workspace(gran)
        # partition outputs of this rank (Q and its own K/V shard), rewritten every step
        p_idx = torch.empty(n_local, dtype=torch.int32, device=dev)
        p_doc = torch.empty(n_local, dtype=torch.int32, device=dev) if w.packed else None
        p_out = [torch.empty((n_local,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev) for t in (gq, gk, gv)]
        ev = {n: [] for n in names}

        def step(timed=None):
            """One step.  timed: None (no events), "calls" (an event pair around every
            call, for the per-call breakdown) or a call name (an event pair around that
            call only)."""
            marks = {}
            c = names.index(timed) if timed in names else -2

            def mark(i):
                if timed == "calls" or i in (c, c + 1):
                    e = TimingEvent()
                    e.record()
                    marks[i] = e

            mark(0)
            C.cpattn_partition(mode, w.seq, w.cp, rank, p_idx, p_doc, [gq, gk, gv], p_out, cu, cu_dev)
            mark(1)
            rs.tile_fwd(edges, parts, workspace=ws_tile)
            mark(2)
            rs.merge(edges, parts, o_t, l_t)
            mark(3)
            rs.stream_fwd(gran, o_s, l_s, workspace=ws_stream)
            mark(4)
            # the dQ pass forms the per-row values D (rowsum(dO * O)) itself, for the
            # dK/dV pass too: the backward as cpattn_bwd runs it
            C.cpattn_bwd_dq_delta(desc, qblk, bsegs, o_s, l_s, g, delta, dq, ws_dq)
            mark(5)
            C.cpattn_bwd_dkdv(desc, qblk, bsegs, l_s, delta, g, dk, dv)
            mark(6)
            for i, n in enumerate(names):
                if i in marks and i + 1 in marks:
                    ev[n].append((marks[i], marks[i + 1]))

        info = dict(rs=rs, edges=edges, split_t=ws_tile is not None, split_s=ws_stream is not None,
                    split_q=ws_dq.numel() > 1, p_idx=p_idx, p_doc=p_doc, p_out=p_out)
        return step, ev, info

    def mean_ms(pairs_of_events):
        return float(np.mean([a.elapsed_time(b) for a, b in pairs_of_events]))

    def timed_run(step, timed=None, warmup=True):
        """K steps bracketed by synchronisations, with an event at each end of the loop:
        (GPU ms per step, wall-clock ms per step).  `timed` adds the step's own events."""
        if warmup:
            for _ in range(args.warmup):
                step()
        torch.cuda.synchronize()
        e0, e1 = TimingEvent(), TimingEvent()
        t0 = time.perf_counter()
        e0.record()
        for _ in range(args.steps):
            step(timed)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps, (time.perf_counter() - t0) * 1e3 / args.steps

    def interleaved_ms(shares, rounds=3, warm_s=1.0):
        """GPU ms per step of every share: warm-up passes over all shares (W steps each)
        for at least ``warm_s`` seconds, then ``rounds`` rounds, each timing K steps of
        every share in turn (as ``timed_run``); the median of the rounds per share."""
        t0 = time.perf_counter()
        while time.perf_counter() - t0 < warm_s:
            for st in shares.values():
                for _ in range(max(args.warmup, 1)):
                    st()
            torch.cuda.synchronize()
        got = {key: [] for key in shares}
        for _ in range(rounds):
            for key, st in shares.items():
                got[key].append(timed_run(st, None, warmup=False)[0])
        return {key: float(np.median(v)) for key, v in got.items()}

    step, ev, info = share_steps(r)
    # the per-call breakdown: an event pair around every call (the events cost GPU time
    # of their own, so this loop is not the headline)
    inst_ms, _ = timed_run(step, "calls")
    ms = {n: mean_ms(ev[n]) for n in names}
    inst_step_ms = sum(ms.values())
    # the headline: whole steps, events only at the ends of the loop and around the
    # dominant kernel's call (the longest call that is one launch)
    split_t, split_s, split_q = info["split_t"], info["split_s"], info["split_q"]
    # the query chunks' merges run as one grouped call: one launch per 8 chunks or 64 parts
    merge_launches, ng, np_ = 0, 0, 0
    for (a_, b_) in info["rs"].q_chunks():
        n = sum(1 for e in info["edges"] if e[0] == (a_, b_))
        if ng == 0 or ng == 8 or np_ + n > 64:
            merge_launches, ng, np_ = merge_launches + 1, 0, 0
        ng, np_ = ng + 1, np_ + n
    launches = {"partition": 1, "tile_fwd": 1 + split_t, "merge": merge_launches, "stream_fwd": 1 + split_s,
                "bwd_dq": 1 + split_q, "bwd_dkdv": 1}
    single = [n for n in names if launches[n] == 1]
    dom = max(single, key=lambda n: ms[n])
    ev[dom] = []
    step_ms, wall_ms = timed_run(step, dom, warmup=False)
    dom_ms = mean_ms(ev[dom])
    # the same step with no event inside the loop (reported beside the headline)
    plain_ms, _ = timed_run(step, None, warmup=False)
    rs, edges = info["rs"], info["edges"]
    # every rank of the 8K share, zigzag and striped (they carry the same or nearly the
    # same visible pairs), timed in interleaved rounds: all shares are built first, then
    # warmed up together, so that no share is timed while the GPU clock climbs back from
    # the idle time of building it (a share timed right after it was built measured
    # ~6 % slower than the same step timed again later)
    other_ranks, striped_cmp = {}, None
    if not w.packed and args.rank is None and len(w.ranks) > 1:
        shares, st_pairs = {("zigzag", r): step}, {}
        for rr in w.ranks:
            if rr != r:
                shares[("zigzag", rr)] = share_steps(rr)[0]
        if len(w.ranks) == w.cp:
            for rr in w.ranks:
                st, _, inf = share_steps(rr, striped=True)
                shares[("striped", rr)] = st
                st_pairs[rr] = int((inf["rs"].q_idx.cpu().numpy().astype(np.int64) + 1).sum())
        share_ms = interleaved_ms(shares)
        other_ranks = {rr: t for (lay, rr), t in share_ms.items() if lay == "zigzag"}
        if st_pairs:
            striped_cmp = ({rr: t for (lay, rr), t in share_ms.items() if lay == "striped"}, st_pairs)
        del shares

    # Rotary embedding fused into the gather (Q and K rotated at the rows' positions, V
    # copied), timed like the plain partition, after the step loop
    rope = C.rope_desc((0, 1), torch.bfloat16, w.d)
    rope_ev = []
    for i in range(args.warmup + args.steps):
        e0, e1 = TimingEvent(), TimingEvent()
        e0.record()
        C.cpattn_partition(part_mode, w.seq, w.cp, r, info["p_idx"], info["p_doc"], [gq, gk, gv], info["p_out"], cu,
                           cu_dev, rope=rope)
        e1.record()
        if i >= args.warmup:
            rope_ev.append((e0, e1))
    torch.cuda.synchronize()
    rope_ms = mean_ms(rope_ev)

    bwd_ms = ms["bwd_dq"] + ms["bwd_dkdv"]
    if w.packed:
        # a row at position p of a document starting at c sees p - c + 1 keys
        pos = rs.q_idx.cpu().numpy().astype(np.int64)
        start = np.asarray(cu, dtype=np.int64)[rs.q_doc.cpu().numpy()]
        pairs = int(np.sum(pos - start + 1))
    else:
        pairs = w.seq * (w.seq + 1) // (2 * w.cp)
    unit = w.d * w.hq * pairs            # (visible pair, head, head-dim element) units
    f_fwd = 4.0 * unit
    f_bwd = 10.0 * unit
    step_flops = 2 * f_fwd + f_bwd
    tflops = lambda f, t_ms: f / (t_ms * 1e-3) / 1e12  # noqa: E731
    gbs = lambda b, t_ms: b / (t_ms * 1e-3) / 1e9  # noqa: E731
    # algorithmic bytes of the bandwidth-bound steps
    elt = 2
    part_bytes = 2 * n_local * (w.hq + 2 * w.hkv) * w.d * elt + 4 * n_local * (1 + w.packed)
    n_parts = [sum(1 for e in edges if e[0] == ch) for ch in rs.q_chunks()]
    merge_bytes = sum(n * (n_local // 2) * w.hq * (w.d * 4 + 4) for n in n_parts) + n_local * w.hq * (w.d * elt + 4)
    # call -> (kernel launches, bound, algorithmic work); the forward calls add a merge
    # launch when their plan splits the KV tiles, the dQ call a sum launch, and the merge
    # call is one grouped launch for the query chunks
    calls = {
        "partition": (launches["partition"], "hbm", part_bytes),
        "tile_fwd": (launches["tile_fwd"], "mfma", f_fwd),
        "merge": (launches["merge"], "hbm", merge_bytes),
        "stream_fwd": (launches["stream_fwd"], "mfma", f_fwd),
        # dQ = dS K, with D formed first; S and dP recomputed, not counted
        "bwd_dq": (launches["bwd_dq"], "mfma", 2.0 * unit),
        "bwd_dkdv": (launches["bwd_dkdv"], "mfma", 8.0 * unit),  # S, dP, dV = P^T dO, dK = dS^T Q
    }
    per_kernel = {}
    for n, (launches, bound, work) in calls.items():
        rate = gbs(work, ms[n]) if bound == "hbm" else tflops(work, ms[n])
        per_kernel[n] = {"us": ms[n] * 1e3, ("GB/s" if bound == "hbm" else "TFLOP/s"): rate,
                         "launches": launches}
    per_kernel["bwd"] = {"us": bwd_ms * 1e3, "TFLOP/s": tflops(f_bwd, bwd_ms)}
    per_kernel["partition_rope"] = {"us": rope_ms * 1e3, "GB/s": gbs(part_bytes, rope_ms), "launches": 2,
                                    "note": "outside the step: Q and K rotated, V copied"}
    # roofline of the dominant kernel, from its events inside the headline loop
    _, bound, work = calls[dom]
    peak = PEAK_BF16_TFLOPS if bound == "mfma" else PEAK_HBM_GBS
    achieved = tflops(work, dom_ms) if bound == "mfma" else gbs(work, dom_ms)
    share = (f"packed-document ({len(cu) - 1} documents, per-document zigzag)" if w.packed
             else "zigzag")
    out = {
        "metric": "causal attn TFLOP/s per rank-share (fwd, bwd) at 1 MI355X; % bf16 MFMA peak",
        "value": round(tflops(step_flops, step_ms), 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall_ms, 4),
        "timing": {"headline": "K whole steps between synchronisations, GPU events at the loop's ends "
                               "and around the dominant kernel's call",
                   "per_kernel": "a separate loop of K steps with an event pair around every call",
                   "instrumented_ms_per_step": round(inst_ms, 4),
                   "sum_of_call_intervals_ms": round(inst_step_ms, 4),
                   "no_event_ms_per_step": round(plain_ms, 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: one {share} rank share, S={w.seq}, cp={w.cp}, rank={r}, "
                               f"Hq={w.hq}, Hkv={w.hkv}, d={w.d}, bf16; KV segments in ring order",
                   "seq_len": w.seq, "cp": w.cp, "rank": r, "hq": w.hq, "hkv": w.hkv, "d": w.d,
                   "visible_pairs_per_head": pairs},
        "pct_bf16_peak": round(100 * tflops(step_flops, step_ms) / PEAK_BF16_TFLOPS, 2),
        "forward_target": {"kernel": "stream_fwd", "frac_of_bf16_peak": round(tflops(f_fwd, ms["stream_fwd"])
                                                                             / PEAK_BF16_TFLOPS, 4),
                           "target_frac": 0.5},
        "per_kernel": {n: {kk: (round(vv, 2) if isinstance(vv, float) else vv) for kk, vv in d_.items()}
                       for n, d_ in per_kernel.items()},
        "bwd_tflops": round(tflops(f_bwd, bwd_ms), 2),
        "fwd_tflops": {"tile+merge": round(tflops(f_fwd, ms["tile_fwd"] + ms["merge"]), 2),
                       "stream": round(tflops(f_fwd, ms["stream_fwd"]), 2)},
        "roofline": {"kernel": KERNEL_OF[dom].format(d=w.d), "call": dom, "bound": bound, "achieved": round(achieved, 2),
                     "peak": peak, "unit": "TFLOP/s" if bound == "mfma" else "GB/s",
                     "frac": round(achieved / peak, 4), "traffic": measured_traffic(dom, args.workload),
                     "algorithmic": work},
    }
    if striped_cmp is not None:
        st_ms, st_pairs = striped_cmp
        zz_ms = dict(other_ranks)
        zz_pairs = pairs
        sp = [st_pairs[x] for x in sorted(st_pairs)]
        out["striped_vs_zigzag"] = {
            "visible_pairs_per_head": {"zigzag": [zz_pairs] * w.cp, "striped": sp},
            "pairs_max_over_min": {"zigzag": 1.0, "striped": round(max(sp) / min(sp), 6)},
            "step_us": {"zigzag": [round(zz_ms[x] * 1e3, 2) for x in sorted(zz_ms)],
                        "striped": [round(st_ms[x] * 1e3, 2) for x in sorted(st_ms)]},
            "note": "same step (partition, tile + merge, stream, backward) per rank; FLOPs differ by the pairs"}
    if other_ranks:
        per_rank = {rr: round(tflops(step_flops, t), 3) for rr, t in other_ranks.items()}
        vals = [per_rank[x] for x in sorted(per_rank)]
        out["per_rank_tflops"] = {"ranks": {str(x): per_rank[x] for x in sorted(per_rank)},
                                  "min": min(vals), "mean": round(sum(vals) / len(vals), 3)}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(q, k, v, w, r, cu)
    print(json.dumps(out), flush=True)


def cpu_baseline(q, k, v, w, r, cu=None, min_seconds=10.0, max_reps=8):
    """The float64 oracle, as it stands, on a bounded sample of the same share: forward and
    backward of the rank's query rows against all keys (for shares longer than 8K an
    evenly spaced subset of 64 rows), repeated until about ``min_seconds`` of CPU work.
    A packed share passes every row's and key's document id with the document mask."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from oracle import attention as OA

    rows = oracle.thd_indices(cu, w.cp, r) if w.packed else oracle.zigzag_indices(w.seq, w.cp, r)
    if w.seq > 8192:
        rows = rows[:: max(1, len(rows) // 64)]
    g = torch.randn((len(rows), w.hq, w.d), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    qr = q[torch.as_tensor(rows)]
    keys = np.arange(w.seq)
    docs = {}
    if w.packed:
        docs = {"q_doc": oracle.thd_doc_ids(cu, rows), "k_doc": oracle.thd_doc_ids(cu, keys),
                "mask": OA.MASK_CAUSAL_DOC}
    reps, t0 = 0, time.perf_counter()
    while True:
        OA.attention_fwd(qr, k, v, rows, keys, **docs)
        OA.attention_bwd(qr, k, v, g, rows, keys, **docs)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds or reps >= max_reps:
            break
    if w.packed:
        pairs = int(np.sum(rows - np.asarray(cu, dtype=np.int64)[docs["q_doc"]] + 1))
    else:
        pairs = int(np.sum(rows + 1))
    flops = reps * (4.0 + 10.0) * w.d * w.hq * pairs
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 numpy oracle, forward + backward of {len(rows)} of the rank's "
                      f"{w.seq // w.cp} query rows against all {w.seq} keys, all {w.hq} heads, "
                      f"{reps} repetition(s); useful FLOPs counted on visible pairs; {dt:.1f} s"}


if __name__ == "__main__":
    main()
