#!/usr/bin/env python3
"""Benchmark one sparse-MoE sub-layer forward pass on one MI355X.

A step is the whole pass: router -> dispatch -> expert up -> expert down
(-> shared experts) -> combine -> routing statistics, on one batch of
synthetic inputs already resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload default]

Steps are timed as one replay of a HIP graph holding the K timed passes back
to back (``ms_per_step_graph_each`` gives K replays of a one-step graph, which
adds the runtime's per-graph launch gap to every step).  Per-call
durations come from HIP events on the stream the kernels run on (torch's
current stream, which every call is given) around K replays of a graph holding
R back-to-back launches of that one call, with the queue kept full so the
events measure the GPU and not host launch latency.  The dominant
kernel is the bf16 grouped GEMM (two launches per step: expert up and expert
down); its roofline figure uses the algorithmic FLOPs of one launch,
2 * rows * d * F for the kept rows, over the measured average launch time.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec at 1 MI355X; grouped-FFN MFMA util %; dispatch GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# Sources that decide which grouped-GEMM kernel runs and what it does: HBM byte
# counters recorded for an older version of them are not reported.
GEMM_SOURCES = ["gemm_bf16_v2.hip", "gemm_tiles.h", "grouped_gemm.hip", "gemm_args.h", "common.h"]
COUNTER_PREFIX = "traffic-json: "

WORKLOADS = {
    "tiny": "TINY", "default": "DEFAULT", "switch_zipf": "SWITCH_ZIPF",
    "fine_shared": "FINE_SHARED", "large_credit": "LARGE_CREDIT",
}


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="default", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--materialise", action="store_true",
                    help="dispatch writes the packed token rows (x_disp) instead of index-only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def copy_calibration():
    """A plain elementwise copy (dst = -src over 1 GiB of fp32, one kernel per
    launch): it reads and writes exactly 1 GiB, so the HBM byte counters of its
    launches give the scale factor for the counters of the other kernels."""
    import torch
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": 4 * n, "copy_bytes_written_per_launch": 4 * n,
                      "launches": 3}), flush=True)


def gemm_source_tag() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_10_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per grouped-GEMM launch (FETCH_SIZE + WRITE_SIZE, each scaled by
    the same counter's reading for a plain copy) from the committed counter
    summaries under profiles/, if one was taken on this workload and on the
    current kernel sources; else None."""
    import glob
    tag = gemm_source_tag()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "gemm_bf16_v2_hbm_counters_*.md"))):
        with open(path) as fh:
            for ln in fh:
                if ln.startswith(COUNTER_PREFIX):
                    rec = json.loads(ln[len(COUNTER_PREFIX):])
                    if rec["workload"] == workload and rec["source_tag"] == tag:
                        return rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"]
    return None


def cpu_baseline(w, seconds: float):
    """Time the CPU oracle on a bounded sample of the same workload."""
    import threadpoolctl
    import oracle
    import synth
    Ts = w.T if w.T <= 4096 else 512
    inp = synth.draw(w.with_(T=Ts))
    info = threadpoolctl.threadpool_info()
    cores = max([i.get("num_threads", 1) for i in info] + [1])
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.forward(inp)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    return {"value": Ts * reps / el, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{reps} full float64 oracle pass(es) over a batch of {Ts} tokens of this workload "
                      f"({el:.1f} s)"}


def main():
    args = _parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this layer has no multi-GPU path (expert "
              "parallelism is designed, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return

    import numpy as np
    import torch
    import synth
    from synth.device import to_torch
    from sparse_mixture_experts_10_amd import MoELayer

    w = getattr(synth, WORKLOADS[args.workload])
    inp = synth.draw(w)
    t = to_torch(inp, "cuda")
    shared = (t["sW1"], t["sb1"], t["sW2"], t["sb2"]) if w.n_shared else None
    layer = MoELayer(t["W_g"], t["W1"], t["b1"], t["W2"], t["b2"], k=w.k, act=w.act,
                     capacity_factor=w.capacity_factor, b_g=t["b_g"], b_sel=t["b_sel"], shared=shared,
                     alpha=w.alpha, beta=w.beta, credit=w.credit, gather_rows=not args.materialise)
    x = t["x"]
    o = layer.allocate(w.T)
    calls = layer.calls(x, o)

    def step():
        layer.forward(x, o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps
    ev = lambda: torch.cuda.Event(enable_timing=True)

    # Whole steps: the K timed steps captured back to back in one HIP graph
    # (as the layers of a model would be) and replayed once between two
    # events, after one untimed replay.  A sleep kernel keeps the GPU busy
    # while the host queues the replay, so the events see the GPU only.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(K):
            step()
    graph.replay()
    torch.cuda.synchronize()
    start, stop = ev(), ev()
    wall0 = time.perf_counter()
    torch.cuda._sleep(int(2.4e9 * 100e-6))
    start.record()
    graph.replay()
    stop.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = start.elapsed_time(stop) / K
    del graph

    # The same K steps as K replays of a one-step graph: each replay adds the
    # runtime's per-graph launch gap (reported alongside, not as the value).
    graph1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph1):
        step()
    for _ in range(args.warmup):
        graph1.replay()
    torch.cuda.synchronize()
    a1, b1 = ev(), ev()
    torch.cuda._sleep(int(2.4e9 * 200e-6 * K))
    a1.record()
    for _ in range(K):
        graph1.replay()
    b1.record()
    torch.cuda.synchronize()
    ms_step_graph_each = a1.elapsed_time(b1) / K
    del graph1

    # Per call: each call captured R times back to back in a graph of its own
    # and replayed K times between two events (queue pre-filled the same way),
    # so the figure is the call's GPU time per launch without host gaps.
    R = 8

    def time_call(fn, budget_us):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(R):
                fn()
        g.replay()
        torch.cuda.synchronize()
        a, b = ev(), ev()
        torch.cuda._sleep(int(2.4e9 * budget_us * 1e-6 * R * K))
        a.record()
        for _ in range(K):
            g.replay()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (K * R)     # microseconds per call

    budget = ms_step * 1e3
    per_call = {name: time_call(fn, budget) for name, fn in calls}
    ms_step_eager = sum(per_call.values()) / 1e3

    # The dispatch on its own (the index-only moe_dispatch call, which the fused
    # routing pass contains), timed the same way, for the dispatch GB/s figure.
    if "dispatch" not in per_call:
        per_call_dispatch = time_call(lambda: layer.dispatch(x, o), budget)
    else:
        per_call_dispatch = per_call["dispatch"]

    # algorithmic work
    T, d, E, k, F = w.T, w.d, w.E, w.k, w.F
    rows = int(o.expert_offset[-1])
    eb = 2 if w.dtype == "bf16" else 4
    gemm_flops = 2.0 * rows * d * F                       # one launch (up or down)
    gemm_us = 0.5 * (per_call["expert_up"] + per_call["expert_down"])
    # algorithmic HBM bytes of one launch, averaged over up and down: rows of A,
    # one expert weight matrix per group, the output rows
    gemm_bytes = 0.5 * ((rows * d + E * F * d + rows * F) + (rows * F + E * d * F + rows * d)) * eb
    achieved = gemm_flops / (gemm_us * 1e-6) / 1e12
    router_bytes = T * d * eb + E * d * 4 + T * E * 4 + T * 4 + 2 * T * k * 4
    # index-only dispatch: read top-k indices, write slot, row and row_token
    # (materialised: plus one read of each kept token row and one write of it)
    dispatch_bytes = T * k * 4 * 3 + rows * 4 + (T * d * eb + rows * d * eb if args.materialise else 0)
    combine_bytes = rows * d * eb + T * d * eb + 2 * T * k * 4 + (T * d * eb if w.n_shared else 0)

    def gbps(b, us):
        return b / (us * 1e-6) / 1e9

    stats_bytes = T * E * 4 + T * 4
    kernels = {}
    if "route" in per_call:
        kernels["route"] = {"us": per_call["route"],
                            "GB/s": gbps(router_bytes + dispatch_bytes + stats_bytes, per_call["route"])}
    else:
        kernels["router"] = {"us": per_call["router"], "GB/s": gbps(router_bytes, per_call["router"])}
    kernels["dispatch"] = {"us": per_call_dispatch, "GB/s": gbps(dispatch_bytes, per_call_dispatch),
                           "note": "index-only moe_dispatch timed on its own" if "route" in per_call else ""}
    kernels.update({
        "expert_up": {"us": per_call["expert_up"],
                      "TFLOP/s": gemm_flops / (per_call["expert_up"] * 1e-6) / 1e12},
        "expert_down": {"us": per_call["expert_down"],
                        "TFLOP/s": gemm_flops / (per_call["expert_down"] * 1e-6) / 1e12},
        "combine": {"us": per_call["combine"], "GB/s": gbps(combine_bytes, per_call["combine"])},
    })
    if "stats" in per_call:
        kernels["stats"] = {"us": per_call["stats"]}
    if w.n_shared:
        kernels["shared"] = {"us": per_call["shared"],
                             "TFLOP/s": 4.0 * T * d * F * w.n_shared / (per_call["shared"] * 1e-6) / 1e12}

    line = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_calls": ms_step_eager,     # sum of the per-call times
        "ms_per_step_graph_each": ms_step_graph_each,   # K replays of a one-step graph
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "d": d, "E": E, "k": k, "F": F, "act": w.act,
                   "capacity_factor": None if w.capacity_factor is None else str(w.capacity_factor),
                   "n_shared": w.n_shared, "kept_rows": rows},
        "roofline": {"bound": "mfma", "kernel": "gemm_bf16_v2_kernel (expert up + down, 2 launches/step)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": counter_traffic(w.name),
                     "algorithmic_bytes": gemm_bytes},
        "mfma_util_pct": 100.0 * achieved / PEAK_BF16_TFLOPS,
        "dispatch_GBps": kernels["dispatch"]["GB/s"],
        "kernels": kernels,
        "wall_s": wall,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
