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

Prints one JSON line (rank 0).  ``--workload s128k`` runs the 128K share instead.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak (published)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E (published)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="s8k", choices=["s8k", "s128k"])
    ap.add_argument("--rank", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU: the other ranks' KV segments are "
                                   "emulated as local buffers; --gpus above 1 is not supported"}))
        sys.exit(2)

    import numpy as np
    import torch

    import workloads
    from context_causal_attention_zigzag_amd.rank_share import (build_rank_share, partition_shard,
                                                                 ring_order)
    import context_causal_attention_zigzag_amd as C

    dev = "cuda"
    w = workloads.WORKLOADS[args.workload]
    r = args.rank
    q, k, v = workloads.full_qkv(w)
    gq, gk, gv = q.to(dev), k.to(dev), v.to(dev)
    gran = "owner" if args.workload == "s8k" else "chunk"
    rs = build_rank_share(gq, gk, gv, w.cp, r)
    n_local = w.seq // w.cp
    g = workloads.randn((n_local, w.hq, w.d), 5, "bf16", 3).to(dev)
    edges, parts = rs.alloc_tile_buffers(gran)
    o_t = torch.empty_like(rs.q)
    l_t = torch.empty((n_local, w.hq), dtype=torch.float32, device=dev)
    o_s = torch.empty_like(rs.q)
    l_s = torch.empty_like(l_t)
    bwd_bufs = rs.alloc_bwd_buffers(gran)
    ws_tile = rs.tile_workspace(edges)
    ws_stream = rs.stream_workspace(gran)
    # partition outputs of this rank (Q and its own K/V shard), rewritten every step
    p_idx = torch.empty(n_local, dtype=torch.int32, device=dev)
    p_out = [torch.empty((n_local,) + tuple(t.shape[1:]), dtype=t.dtype, device=dev) for t in (gq, gk, gv)]

    names = ["partition", "tile_fwd", "merge", "stream_fwd", "bwd"]
    ev = {n: [] for n in names}

    def step(timed):
        marks = []

        def mark():
            if timed:
                e = torch.cuda.Event(enable_timing=True)
                e.record()
                marks.append(e)

        mark()
        C.cpattn_partition(C.PART_ZIGZAG, w.seq, w.cp, r, p_idx, None, [gq, gk, gv], p_out)
        mark()
        rs.tile_fwd(edges, parts, workspace=ws_tile)
        mark()
        rs.merge(edges, parts, o_t, l_t)
        mark()
        rs.stream_fwd(gran, o_s, l_s, workspace=ws_stream)
        mark()
        rs.bwd(o_s, l_s, g, bwd_bufs, gran)
        mark()
        if timed:
            for i, n in enumerate(names):
                ev[n].append((marks[i], marks[i + 1]))

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step(True)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0

    ms = {n: float(np.mean([a.elapsed_time(b) for a, b in ev[n]])) for n in names}
    step_ms = sum(ms.values())
    pairs = w.seq * (w.seq + 1) // (2 * w.cp)
    f_fwd = 4.0 * w.d * w.hq * pairs
    f_bwd = 10.0 * w.d * w.hq * pairs
    step_flops = 2 * f_fwd + f_bwd
    tflops = lambda f, t_ms: f / (t_ms * 1e-3) / 1e12  # noqa: E731
    # algorithmic bytes of the bandwidth-bound steps
    elt = 2
    part_bytes = 2 * n_local * (w.hq + 2 * w.hkv) * w.d * elt + 4 * n_local
    n_parts = [sum(1 for e in edges if e[0] == ch) for ch in rs.q_chunks()]
    merge_bytes = sum(n * (n_local // 2) * w.hq * (w.d * 4 + 4) for n in n_parts) + n_local * w.hq * (w.d * elt + 4)
    per_kernel = {
        "partition": {"us": ms["partition"] * 1e3, "GB/s": part_bytes / (ms["partition"] * 1e-3) / 1e9},
        "tile_fwd": {"us": ms["tile_fwd"] * 1e3, "TFLOP/s": tflops(f_fwd, ms["tile_fwd"])},
        "merge": {"us": ms["merge"] * 1e3, "GB/s": merge_bytes / (ms["merge"] * 1e-3) / 1e9},
        "stream_fwd": {"us": ms["stream_fwd"] * 1e3, "TFLOP/s": tflops(f_fwd, ms["stream_fwd"])},
        "bwd": {"us": ms["bwd"] * 1e3, "TFLOP/s": tflops(f_bwd, ms["bwd"])},
    }
    dom = max(["tile_fwd", "stream_fwd", "bwd"], key=lambda n: ms[n])
    dom_flops = f_bwd if dom == "bwd" else f_fwd
    achieved = tflops(dom_flops, ms[dom])
    out = {
        "metric": "causal attn TFLOP/s per rank-share (fwd, bwd) at 1 MI355X; % bf16 MFMA peak",
        "value": round(tflops(step_flops, step_ms), 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 4),
        "wall_ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: one zigzag rank share, S={w.seq}, cp={w.cp}, rank={r}, "
                               f"Hq={w.hq}, Hkv={w.hkv}, d={w.d}, bf16; KV segments in ring order",
                   "seq_len": w.seq, "cp": w.cp, "rank": r, "hq": w.hq, "hkv": w.hkv, "d": w.d,
                   "visible_pairs_per_head": pairs},
        "pct_bf16_peak": round(100 * tflops(step_flops, step_ms) / PEAK_BF16_TFLOPS, 2),
        "per_kernel": {n: {kk: round(vv, 2) for kk, vv in d_.items()} for n, d_ in per_kernel.items()},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": None},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(q, k, v, w, r)
    print(json.dumps(out), flush=True)


def cpu_baseline(q, k, v, w, r):
    """The float64 oracle, as it stands, on a bounded sample of the same share: forward and
    backward of every 2nd local query row against all keys."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from oracle import attention as OA

    rows = oracle.zigzag_indices(w.seq, w.cp, r)[::2]
    g = torch.randn((len(rows), w.hq, w.d), generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    t0 = time.perf_counter()
    OA.attention_fwd(q[torch.as_tensor(rows)], k, v, rows, np.arange(w.seq))
    OA.attention_bwd(q[torch.as_tensor(rows)], k, v, g, rows, np.arange(w.seq))
    dt = time.perf_counter() - t0
    pairs = int(np.sum(rows + 1))
    flops = (4.0 + 10.0) * w.d * w.hq * pairs
    threads = max([x.get("num_threads", 1) for x in threadpool_info()] or [1])
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": f"float64 numpy oracle, forward + backward of {len(rows)} of the rank's "
                      f"{w.seq // w.cp} query rows (every 2nd) against all {w.seq} keys, all {w.hq} heads; "
                      f"useful FLOPs counted on visible pairs; {dt:.1f} s"}


if __name__ == "__main__":
    main()
