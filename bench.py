#!/usr/bin/env python3
"""Benchmark of the routed-experts MoE decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the MXFP8
plan of x (moe_plan), the unit table (moe_group) and the persistent experts kernel
(moe_experts_run: FC1 -> SwiGLU -> hidden requant -> FC2 -> BF16 rows).  Inputs are
resident in HBM before the timed region starts.  Each step reads a different weight
replica (>= 1 GiB rotated) so the 256 MB Infinity Cache cannot serve repeated weights.
Steps are captured in a HIP graph (torch.cuda.CUDAGraph) and replayed; the timed
region is bracketed by synchronizations and HIP events on the launch stream.

Prints ONE JSON line (rank 0): µs per layer of the named workload, plus the roofline
of the dominant kernel (experts: algorithmic bytes / its average duration measured
with HIP events over graph replays of that kernel alone) and the CPU oracle timed on
the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s


def _unique_weight_bytes(ids, w) -> int:
    import numpy as np
    import workloads
    n = len(np.unique(ids))
    return n * workloads.expert_weight_bytes(w.D, w.I)


def measure(name: str, steps: int, warmup: int, *, graph_steps: int = 24, log=print) -> dict:
    import numpy as np
    import torch

    import workloads
    from moe_routed_expert_mx_amd.layer import MoeLayer

    d = workloads.generate(name)
    w = d["workload"]
    per_expert = workloads.expert_weight_bytes(w.D, w.I)
    R = max(2, math.ceil((1 << 30) / (w.E * per_expert)))
    layer = MoeLayer(d["w13"], d["s13"], d["w2"], d["s2"], B_max=w.B, topk=w.K, device="cuda", replicas=R)
    x = torch.from_numpy(d["x"]).cuda()
    ids = torch.from_numpy(d["ids"]).cuda()
    out = layer.out_buffer(w.B)
    G = max(graph_steps // R, 1) * R

    for i in range(warmup):
        layer.forward(x, ids, out, replica=i % R)
    torch.cuda.synchronize()

    # whole step (plan + units + experts), captured G steps per graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(G):
            layer.forward(x, ids, out, replica=i % R)
    for _ in range(2):
        g.replay()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(steps / G))
    stream = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(reps):
        g.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    step_us = t0.elapsed_time(t1) * 1e3 / (reps * G)

    # dominant kernel alone: the experts kernel on the plan/units of the last step
    ge = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ge):
        for i in range(G):
            layer.experts(w.B, out, replica=i % R)
    ge.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        ge.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    experts_us = e0.elapsed_time(e1) * 1e3 / (reps * G)

    uniq = _unique_weight_bytes(d["ids"], w)
    io_bytes = w.B * w.D * 2 + w.B * w.K * 4 + w.B * w.K * w.D * 2  # x, ids, out
    plan_bytes = w.B * w.D * 33 // 32
    experts_bytes = uniq + plan_bytes + w.B * w.K * w.D * 2          # weights + plan read + out
    res = {
        "workload": name, "B": w.B, "E": w.E, "topk": w.K, "D": w.D, "I": w.I,
        "distinct_experts": int(len(np.unique(d["ids"]))), "replicas": R, "graph_steps": G,
        "step_us": step_us, "experts_us": experts_us,
        "routes_per_s": w.B * w.K / (step_us * 1e-6),
        "unique_weight_bytes": uniq, "step_bytes": uniq + io_bytes,
        "experts_alg_bytes": experts_bytes,
        "step_gbs": uniq / (step_us * 1e-6) / 1e9,
        "experts_gbs": experts_bytes / (experts_us * 1e-6) / 1e9,
    }
    log(json.dumps({"config_detail": res}), file=sys.stderr)
    del g, ge, layer
    torch.cuda.empty_cache()
    return res


def cpu_baseline(name: str, budget_s: float = 10.0) -> dict:
    """The oracle (plan + per-route experts) on the host cores, repeated over the whole
    layer until `budget_s` of wall time; a bounded sample for the big layers."""
    import numpy as np

    import oracle
    import workloads

    d = workloads.generate(name)
    w = d["workload"]
    threads = max(1, len(os.sched_getaffinity(0)))
    R = w.B * w.K
    # one route takes ~6*I*D flops in FP64 with exactness checks; sample <= 256 routes
    routes = None
    if R > 256:
        routes = np.random.default_rng(0).choice(R, 256, replace=False).astype(np.int32)
    n_routes = R if routes is None else len(routes)
    runs = 0
    t_start = time.perf_counter()
    while True:
        codes, scales = oracle.plan(d["x"])
        oracle.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                       hidden_floor=oracle.default_hidden_floor(w.I), routes=routes, nthreads=threads,
                       want_hidden=False)
        runs += 1
        el = time.perf_counter() - t_start
        if el >= budget_s or runs >= 1000:
            break
    per_route_s = el / (runs * n_routes)
    layer_us = per_route_s * R * 1e6
    sample = (f"{runs} oracle run(s) of plan + {n_routes} of {R} routes "
              f"({'all' if routes is None else 'a seeded random sample'}), {el:.1f} s wall, scaled to the layer")
    return {"value": layer_us, "unit": "us", "cores": threads, "kind": "oracle", "sample": sample}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=240)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="decode_b1")
    ap.add_argument("--all", action="store_true", help="also time the other four workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU; --gpus {args.gpus} is not supported "
              "(the path shards by TP/EP across GPUs, see the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    names = workloads.ORDER if args.all else [args.workload]
    results = {n: measure(n, args.steps, args.warmup) for n in names}
    main_res = results[args.workload]
    cpu = None if args.no_cpu_baseline else cpu_baseline(args.workload, args.cpu_budget)
    line = {
        "metric": "us per MoE layer & achieved HBM GB/s (% of peak), B=1..256",
        "value": round(main_res["step_us"], 3),
        "unit": "us",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(main_res["step_us"] / 1e3, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp4xfp8->f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "B": main_res["B"], "E": main_res["E"], "topk": main_res["topk"],
                   "D": main_res["D"], "I": main_res["I"], "parallelism": "single GPU (one TP shard)"},
        "routes_per_s": round(main_res["routes_per_s"], 1),
        "hbm_gbs_unique_weights": round(main_res["step_gbs"], 1),
        "hbm_frac_of_peak": round(main_res["step_gbs"] / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": "experts_kernel",
            "achieved": round(main_res["experts_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(main_res["experts_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": None,
            "avg_us": round(main_res["experts_us"], 3),
        },
        "cpu_baseline": cpu,
    }
    if args.all:
        line["per_workload"] = {n: {"us": round(r["step_us"], 3), "experts_us": round(r["experts_us"], 3),
                                    "routes_per_s": round(r["routes_per_s"], 1),
                                    "gbs_unique": round(r["step_gbs"], 1),
                                    "frac": round(r["step_gbs"] / HBM_PEAK_GBS, 4)} for n, r in results.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
