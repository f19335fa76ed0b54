#!/usr/bin/env python3
"""Benchmark one sparse-MoE sub-layer forward pass on one MI355X.

A step is the whole pass: router -> dispatch -> expert up -> expert down
(-> shared experts) -> combine -> routing statistics (-> credit), on one batch
of synthetic inputs already resident in HBM.  Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload large_credit]

The default workload is the largest one that the layer is measured on: 32768
tokens, d 4096, 128 experts, top-8, expert width 1536, GELU, bf16, dropless,
with the activation-weighted credit.

Steps are timed as one replay of a HIP graph holding the K timed passes back
to back; ``ms_per_step_graph_each`` gives K replays of a one-step graph (each
adds the runtime's launch gap), ``ms_per_step_flushed`` the median of K steps
each after a 1 GiB write that evicts the caches (outside the timed region).
Per-call durations come from HIP events on the stream the kernels run on
(torch's current stream, which every call is given) around K replays of a
graph holding R back-to-back launches of that one call, with the queue kept
full so the events measure the GPU and not host launch latency.

The dominant kernel is the bf16 grouped GEMM (two launches per step: expert
up and expert down).  Its roofline takes the binding resource of one launch:
the algorithmic flops 2 rows d F against the dense bf16 MFMA peak, or the
algorithmic bytes (gathered A rows, every expert's weights, output rows)
against the HBM peak, whichever takes longer; ``achieved`` is that work over
the measured average launch time.  On-box ceilings from the library's own
copy, streaming-read and MFMA-loop kernels are reported beside the published
peaks.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer fwd tokens/sec at 1 MI355X; grouped-FFN MFMA util %; dispatch GB/s"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E

# Sources that decide which grouped-GEMM kernel runs and what it does: HBM byte
# counters recorded for an older version of them are not reported.
GEMM_SOURCES = ["gemm_bf16_v2.hip", "gemm_bf16_persist.hip", "gemm_tiles.h", "grouped_gemm.hip", "gemm_args.h",
                "common.h", "lds_ring.h"]
COUNTER_PREFIX = "traffic-json: "

WORKLOADS = {
    "tiny": "TINY", "default": "DEFAULT", "switch_zipf": "SWITCH_ZIPF",
    "fine_shared": "FINE_SHARED", "large_credit": "LARGE_CREDIT",
}
# workloads whose grouped-GEMM utilisation is reported beside the headline
EXTRA = ("switch_zipf", "fine_shared")


def _parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[1])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="large_credit", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the grouped-GEMM figures of the switch and fine-grained workloads")
    ap.add_argument("--materialise", action="store_true",
                    help="dispatch writes the packed token rows (x_disp) instead of index-only")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run the library's copy kernel over 1 GiB (reference for HBM byte counters)")
    return ap.parse_args()


def _ev():
    import torch
    return torch.cuda.Event(enable_timing=True)


def copy_calibration():
    """The library's copy kernel over 1 GiB, three launches: it reads and writes
    exactly 1 GiB, so the HBM byte counters of its launches give the scale
    factor for the counters of the other kernels."""
    import torch
    from sparse_mixture_experts_10_amd import api
    n = 1 << 30
    src = torch.zeros(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        api.moe_calib_copy(src, dst, n)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 3}),
          flush=True)


def ceilings():
    """On-box rates of the library's calibration kernels: a 2 GiB -> 2 GiB
    copy (read + write bytes per second), a 4 GiB streaming read, and the
    MFMA loop (dense bf16).  Best of five launches each."""
    import torch
    from sparse_mixture_experts_10_amd import api

    def best(fn, reps=5):
        ts = []
        for _ in range(reps):
            a, b = _ev(), _ev()
            torch.cuda._sleep(int(2.4e9 * 50e-6))
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(b) * 1e-3)
        return min(ts)

    n = 2 << 30
    src = torch.zeros(2 * n, dtype=torch.uint8, device="cuda")
    dst = torch.empty(n, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    api.moe_calib_copy(src, dst, n)
    t_copy = best(lambda: api.moe_calib_copy(src, dst, n))
    t_read = best(lambda: api.moe_calib_read(src, 2 * n, sink))
    del src, dst
    fsink = torch.zeros(1, dtype=torch.float32, device="cuda")
    blocks, iters = 2048, 2048
    flops = api.moe_calib_mfma(blocks, iters, fsink)
    t_mfma = best(lambda: api.moe_calib_mfma(blocks, iters, fsink))
    return {"copy_GBps": 2 * n / t_copy / 1e9, "read_GBps": 2 * n / t_read / 1e9,
            "mfma_bf16_TFLOPs": flops / t_mfma / 1e12,
            "note": "library calibration kernels (include/moe_calib.h), best of 5 launches; copy counts "
                    "read + write bytes"}


def gemm_source_tag() -> str:
    """Hash of the grouped GEMM's sources with comments and blank space taken
    out, so a counter summary stays matched through comment-only edits."""
    import hashlib, re
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "sparse_mixture_experts_10_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload: str):
    """HBM bytes per grouped-GEMM launch (FETCH_SIZE + WRITE_SIZE, each scaled by
    the same counter's reading for a plain copy) from the committed counter
    summaries under profiles/, if one was taken on this workload and on the
    current kernel sources; else None."""
    import glob
    tag = gemm_source_tag()
    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", "*hbm_counters*.md"))):
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


def build(w, materialise=False):
    import synth
    from synth.device import to_torch
    from sparse_mixture_experts_10_amd import MoELayer
    inp = synth.draw(w)
    t = to_torch(inp, "cuda")
    shared = (t["sW1"], t["sb1"], t["sW2"], t["sb2"]) if w.n_shared else None
    layer = MoELayer(t["W_g"], t["W1"], t["b1"], t["W2"], t["b2"], k=w.k, act=w.act,
                     capacity_factor=w.capacity_factor, b_g=t["b_g"], b_sel=t["b_sel"], shared=shared,
                     alpha=w.alpha, beta=w.beta, credit=w.credit, gather_rows=not materialise)
    return layer, t["x"]


def time_graph(fn, K, budget_us, R=1):
    """GPU microseconds per call of fn: R back-to-back calls captured in one
    graph, replayed K times between two events, after one untimed replay; a
    sleep kernel keeps the queue full while the host enqueues the replays."""
    import torch
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(R):
            fn()
    g.replay()
    torch.cuda.synchronize()
    a, b = _ev(), _ev()
    torch.cuda._sleep(int(2.4e9 * min(budget_us * 1e-6 * R * K, 0.5)))
    a.record()
    for _ in range(K):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    del g
    return a.elapsed_time(b) * 1e3 / (K * R)


def gemm_figures(w, rows, up_us, down_us):
    """Algorithmic work of one grouped-GEMM launch (mean of up and down) and
    its binding resource at the published peaks."""
    T, d, E, k, F = w.T, w.d, w.E, w.k, w.F
    eb = 2 if w.dtype == "bf16" else 4
    flops = 2.0 * rows * d * F
    bytes_ = 0.5 * ((rows * d + E * F * d + rows * F) + (rows * F + E * d * F + rows * d)) * eb
    us = 0.5 * (up_us + down_us)
    t_mfma = flops / (PEAK_BF16_TFLOPS * 1e12)
    t_hbm = bytes_ / (PEAK_HBM_GBPS * 1e9)
    tflops = flops / (us * 1e-6) / 1e12
    gbps = bytes_ / (us * 1e-6) / 1e9
    return {"flops": flops, "bytes": bytes_, "us": us, "TFLOP/s": tflops, "GB/s": gbps,
            "bound": "mfma" if t_mfma >= t_hbm else "hbm",
            "mfma_util_pct": 100.0 * tflops / PEAK_BF16_TFLOPS, "hbm_frac": gbps / PEAK_HBM_GBPS,
            "roofline_frac": max(t_mfma, t_hbm) / (us * 1e-6)}


def extra_workload(name, K):
    """Grouped-GEMM utilisation and step time of another workload (parity
    cases of the same layer; reported beside the headline)."""
    import torch
    import synth
    w = getattr(synth, WORKLOADS[name])
    layer, x = build(w)
    o = layer.allocate(w.T)
    for _ in range(3):
        layer.forward(x, o)
    torch.cuda.synchronize()
    step_ms = time_graph(lambda: layer.forward(x, o), 1, 1e4, R=K) / 1e3
    per = {n: time_graph(fn, K, 1e3 * step_ms, R=4) for n, fn in layer.calls(x, o)}
    rows = int(o.expert_offset[-1])
    g = gemm_figures(w, rows, per["expert_up"], per["expert_down"])
    out = {"workload": w.name, "ms_per_step": step_ms, "tokens_per_s": w.T / (step_ms * 1e-3),
           "kept_rows": rows, "gemm_bound": g["bound"], "gemm_TFLOPs": g["TFLOP/s"],
           "gemm_mfma_util_pct": g["mfma_util_pct"], "gemm_GBps": g["GB/s"], "gemm_hbm_frac": g["hbm_frac"],
           "gemm_roofline_frac": g["roofline_frac"],
           "us": {n: round(v, 2) for n, v in per.items()}}
    del layer, x, o
    torch.cuda.empty_cache()
    return out


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

    import torch
    import synth
    from sparse_mixture_experts_10_amd import api

    w = getattr(synth, WORKLOADS[args.workload])
    layer, x = build(w, args.materialise)
    o = layer.allocate(w.T)
    calls = layer.calls(x, o)

    def step():
        layer.forward(x, o)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    K = args.steps

    # Whole steps: the K timed steps captured back to back in one HIP graph
    # (as the layers of a model would be) and replayed once between two
    # events, after one untimed replay.
    wall0 = time.perf_counter()
    ms_step = time_graph(step, 1, 1e4, R=K) / 1e3
    wall = time.perf_counter() - wall0

    # The same K steps as K replays of a one-step graph: each replay adds the
    # runtime's per-graph launch gap (reported alongside, not as the value).
    ms_step_graph_each = time_graph(step, K, 1e3 * ms_step, R=1) / 1e3

    # Cache-flushed steps: before each, a 1 GiB write (the library's copy
    # kernel) evicts the L2s and the 256 MB last-level cache; only the step
    # is between the events.  Median over K steps.
    flush_src = torch.zeros(1 << 30, dtype=torch.uint8, device="cuda")
    flush_dst = torch.empty_like(flush_src)
    g1 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g1):
        step()
    g1.replay()
    torch.cuda.synchronize()
    evs = []
    torch.cuda._sleep(int(2.4e9 * min(K * (1e-3 * ms_step + 400e-6), 0.5)))
    for _ in range(K):
        api.moe_calib_copy(flush_src, flush_dst, 1 << 30)
        a, b = _ev(), _ev()
        a.record()
        g1.replay()
        b.record()
        evs.append((a, b))
    torch.cuda.synchronize()
    flushed = [a.elapsed_time(b) for a, b in evs]
    del g1, flush_src, flush_dst

    # Per call: each call captured R times back to back in a graph of its own
    # and replayed K times between two events.
    budget = ms_step * 1e3
    per_call = {name: time_graph(fn, K, budget, R=8) for name, fn in calls}
    ms_step_eager = sum(per_call.values()) / 1e3

    # Dispatch on its own: the index-only call (what the routing pass
    # contains), and the materialised gather (token rows copied to expert
    # order), whose bytes are the dispatch's data movement.  The timed step
    # gathers the rows inside the expert-up GEMM's loads instead.
    T, d, E, k, F = w.T, w.d, w.E, w.k, w.F
    eb = 2 if w.dtype == "bf16" else 4
    rows = int(o.expert_offset[-1])
    i32 = dict(dtype=torch.int32, device="cuda")
    d_cnt, d_off = torch.empty(E, **i32), torch.empty(E + 1, **i32)
    d_slot, d_row = torch.empty(T, k, **i32), torch.empty(T, k, **i32)
    d_rt = torch.empty(max(o.max_rows, 1), **i32)
    d_ws = torch.empty(max(api.moe_workspace_bytes(api.OP_DISPATCH, T=T, E=E), 256), dtype=torch.uint8,
                       device="cuda")
    x_disp = torch.empty(max(o.max_rows, 1), d, dtype=x.dtype, device="cuda")
    us_index = time_graph(lambda: api.moe_dispatch(o.topk_idx, E, o.capacity, None, d_cnt, d_off, d_slot, d_row,
                                                   d_rt, None, d_ws), K, budget, R=8)
    us_gather = time_graph(lambda: api.moe_dispatch(o.topk_idx, E, o.capacity, x, d_cnt, d_off, d_slot, d_row,
                                                    d_rt, x_disp, d_ws), K, budget, R=8)
    del x_disp
    index_bytes = T * k * 4 * 3 + rows * 4
    gather_bytes = index_bytes + 2 * rows * d * eb

    g = gemm_figures(w, rows, per_call["expert_up"], per_call["expert_down"])
    router_bytes = T * d * eb + E * d * 4 + T * E * 4 + T * 4 + 2 * T * k * 4
    stats_bytes = T * E * 4 + T * 4
    combine_bytes = rows * d * eb + T * d * eb + 2 * T * k * 4 + (T * d * eb if w.n_shared else 0)

    def hbm(b, us):
        gb = b / (us * 1e-6) / 1e9
        return {"us": us, "GB/s": gb, "hbm_frac": gb / PEAK_HBM_GBPS, "bytes": b}

    kernels = {}
    if "route" in per_call:
        kernels["route"] = hbm(router_bytes + index_bytes + stats_bytes, per_call["route"])
    else:
        kernels["router"] = hbm(router_bytes, per_call["router"])
    kernels["dispatch"] = dict(hbm(gather_bytes, us_gather),
                               note="materialised gather: index build plus token rows copied to expert order")
    kernels["dispatch_index_only"] = {"us": us_index, "bytes": index_bytes}
    kernels["expert_up"] = {"us": per_call["expert_up"],
                            "TFLOP/s": g["flops"] / (per_call["expert_up"] * 1e-6) / 1e12}
    kernels["expert_down"] = {"us": per_call["expert_down"],
                              "TFLOP/s": g["flops"] / (per_call["expert_down"] * 1e-6) / 1e12}
    kernels["combine"] = hbm(combine_bytes, per_call["combine"])
    if "stats" in per_call:
        kernels["stats"] = {"us": per_call["stats"]}
    if w.n_shared:
        kernels["shared"] = {"us": per_call["shared"],
                             "TFLOP/s": 4.0 * T * d * F * w.n_shared / (per_call["shared"] * 1e-6) / 1e12}

    if g["bound"] == "mfma":
        roof = {"bound": "mfma", "achieved": g["TFLOP/s"], "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": g["GB/s"], "peak": PEAK_HBM_GBPS, "unit": "GB/s"}
    roof.update({"frac": roof["achieved"] / roof["peak"], "traffic": counter_traffic(w.name),
                 "kernel": "grouped bf16 GEMM, expert up + down (2 launches/step; gemm_bf16_persist_kernel "
                           "on 256 x 256 tiles, gemm_bf16_v2_kernel on the other tile shapes)",
                 "algorithmic_bytes": g["bytes"], "algorithmic_flops": g["flops"]})

    line = {
        "metric": METRIC,
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_calls": ms_step_eager,                 # sum of the per-call times
        "ms_per_step_graph_each": ms_step_graph_each,       # K replays of a one-step graph
        "ms_per_step_flushed": statistics.median(flushed),  # each step after a 1 GiB cache-evicting write
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "T": T, "d": d, "E": E, "k": k, "F": F, "act": w.act,
                   "capacity_factor": None if w.capacity_factor is None else str(w.capacity_factor),
                   "n_shared": w.n_shared, "credit": w.credit, "kept_rows": rows},
        "roofline": roof,
        "mfma_util_pct": g["mfma_util_pct"],
        "dispatch_GBps": kernels["dispatch"]["GB/s"],
        "kernels": kernels,
        "wall_s": wall,
    }
    del layer, x, o, calls
    torch.cuda.empty_cache()
    line["ceilings"] = ceilings()
    if not args.no_extra and args.workload == "large_credit":
        line["extra_workloads"] = {n: extra_workload(n, min(K, 10)) for n in EXTRA}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
