#!/usr/bin/env python3
"""Benchmark of the routed-experts MoE decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the MXFP8
plan of x, the unit table and the persistent experts kernel (FC1 -> SwiGLU -> hidden
requant -> FC2 -> BF16 rows).  For B <= 8 that is one moe_decode_run launch (the
kernel quantizes and routes the batch itself); for larger batches two calls,
moe_plan_group (the plan of x and the unit table) + moe_experts_run.  Inputs are
resident in HBM before the timed region starts.  Each step reads a different weight
replica (>= 1 GiB rotated) so the 256 MB Infinity Cache cannot serve repeated weights.
Steps are captured in a HIP graph (torch.cuda.CUDAGraph) and replayed; the timed
region is bracketed by synchronizations and HIP events on the launch stream.

Prints ONE JSON line (rank 0): µs per layer of the named workload, plus the roofline
of the dominant kernel (experts: algorithmic bytes / its average duration measured
with HIP events over graph replays of that kernel alone), the CPU oracle timed on
the host cores on a bounded sample of the same workload, and the weighted top-k
combine (moe_combine) of the step's rows timed alone (it follows the step; it is not
part of it).
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
KERNEL_SRC = os.path.join(ROOT, "moe_routed_expert_mx_amd", "csrc", "moe_mx.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "experts_kernel_traffic.json")


def kernel_hash() -> str:
    """sha256[:16] of the kernel source's code: line comments and blank lines are left
    out, so that a change of comments alone keeps the recorded traffic valid."""
    import hashlib
    import re
    with open(KERNEL_SRC, encoding="utf-8") as f:
        lines = (re.sub(r"//.*$", "", ln).rstrip() for ln in f)
        code = "\n".join(ln for ln in lines if ln)
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM-side bytes per experts-kernel launch from the committed rocprofv3 PMC summary
    (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None when there
    is none for this workload or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha256_16") != kernel_hash():
        return None
    w = t.get("workloads", {}).get(workload)
    return None if w is None else w.get("bytes_per_launch")


def copy_calibration(mb: int) -> None:
    """A plain device copy of `mb` MiB (a torch elementwise kernel), three times: the
    known-size reference that scales the PMC byte counters."""
    import torch
    n = mb << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 3}), file=sys.stderr)


def _unique_weight_bytes(ids, w) -> int:
    import numpy as np
    import workloads
    n = len(np.unique(ids))
    return n * workloads.expert_weight_bytes(w.D, w.I)


def measure(name: str, steps: int, warmup: int, *, graph_steps: int = 48, eager: bool = False, path: str = "auto",
            exchange: int | None = None, log=print) -> dict:
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
    rw = torch.from_numpy(d["weights"]).cuda()
    out = layer.out_buffer(w.B)
    y = torch.empty(w.B, w.D, dtype=torch.bfloat16, device="cuda")
    # steps per graph: the largest divisor of `steps` up to graph_steps, so that exactly
    # `steps` steps are timed
    G = max(gs for gs in range(1, min(graph_steps, steps) + 1) if steps % gs == 0)
    decode = w.B <= MoeLayer.DECODE_MAX and (path == "decode" or (path == "auto" and MoeLayer.AUTO_DECODE))
    form = "decode" if decode else "grouped"
    xo = {"exchange": exchange} if (decode and exchange is not None) else {}

    for i in range(warmup):
        layer.forward(x, ids, out, replica=i % R, path=form, **xo)
    torch.cuda.synchronize()

    reps = steps // G
    stream = torch.cuda.current_stream()
    g = ge = gc = None
    if not eager:
        # whole step (plan + units + experts), captured G steps per graph
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(G):
                layer.forward(x, ids, out, replica=i % R, path=form, **xo)
        # the dominant kernel alone: the experts kernel on the plan/units of the last step
        # (the decode form's step is that one kernel)
        ge = torch.cuda.CUDAGraph()
        with torch.cuda.graph(ge):
            for i in range(G):
                if decode:
                    layer.forward(x, ids, out, replica=i % R, path=form, **xo)
                else:
                    layer.experts(w.B, out, replica=i % R)
        # the weighted top-k combine of the step's rows (outside the step)
        gc = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gc):
            for i in range(G):
                layer.combine(out, rw, y)
        for _ in range(2):
            g.replay()
            ge.replay()
            gc.replay()
        layer.forward(x, ids, out, path=form, **xo)  # plan and units of this batch for the experts-only graph
        torch.cuda.synchronize()

    def timed(run_all) -> float:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        run_all()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / (reps * G)

    def steps_eager():
        for i in range(reps * G):
            layer.forward(x, ids, out, replica=i % R, path=form, **xo)

    def experts_eager():
        for i in range(reps * G):
            if decode:
                layer.forward(x, ids, out, replica=i % R, path=form, **xo)
            else:
                layer.experts(w.B, out, replica=i % R)

    def combine_eager():
        for i in range(reps * G):
            layer.combine(out, rw, y)

    step_us = timed(steps_eager if eager else (lambda: [g.replay() for _ in range(reps)]))
    experts_us = timed(experts_eager if eager else (lambda: [ge.replay() for _ in range(reps)]))
    combine_us = timed(combine_eager if eager else (lambda: [gc.replay() for _ in range(reps)]))
    combine_bytes = w.B * w.K * w.D * 2 + w.B * w.K * 4 + w.B * w.D * 2  # rows, weights, y

    uniq = _unique_weight_bytes(d["ids"], w)
    io_bytes = w.B * w.D * 2 + w.B * w.K * 4 + w.B * w.K * w.D * 2  # x, ids, out
    plan_bytes = w.B * w.D * 33 // 32
    # weights + the activations the kernel reads (the plan, or x and ids in the decode
    # form) + output rows
    act_bytes = w.B * w.D * 2 + w.B * w.K * 4 if decode else plan_bytes
    experts_bytes = uniq + act_bytes + w.B * w.K * w.D * 2
    # the decode form's default exchange runs decode_whole_kernel (whole-K hidden blocks)
    # for batches within its limits (at most 128 distinct experts); the others run
    # experts_kernel
    whole = decode and exchange in (None, 0) and min(w.E, w.B * w.K) <= 128
    res = {
        "workload": name, "form": form,
        "kernel": "decode_whole_kernel" if whole else ("experts_kernel (decode form)" if decode else "experts_kernel"), "B": w.B, "E": w.E, "topk": w.K, "D": w.D, "I": w.I,
        "distinct_experts": int(len(np.unique(d["ids"]))), "replicas": R, "graph_steps": G,
        "step_us": step_us, "experts_us": experts_us,
        "routes_per_s": w.B * w.K / (step_us * 1e-6),
        "unique_weight_bytes": uniq, "step_bytes": uniq + io_bytes,
        "experts_alg_bytes": experts_bytes,
        "step_gbs": uniq / (step_us * 1e-6) / 1e9,
        "experts_gbs": experts_bytes / (experts_us * 1e-6) / 1e9,
        "combine_us": combine_us, "combine_alg_bytes": combine_bytes,
        "combine_gbs": combine_bytes / (combine_us * 1e-6) / 1e9,
    }
    log(json.dumps({"config_detail": res}), file=sys.stderr)
    del g, ge, gc, layer
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
        if el >= budget_s:
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
    ap.add_argument("--eager", action="store_true", help="launch kernels directly instead of replaying HIP graphs")
    ap.add_argument("--exchange", type=int, default=None,
                    help="decode form: FC1 -> FC2 exchange variant (moe_run_opts_t.exchange); default: the library's")
    ap.add_argument("--path", default="auto", choices=("auto", "decode", "grouped"),
                    help="step form for B <= 8: one decode launch, the two-call grouped form, or auto "
                         "(larger batches always use the grouped form)")
    ap.add_argument("--copy-mb", type=int, default=0,
                    help="also run a plain device copy of this many MiB (PMC calibration)")
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
    if args.copy_mb > 0:
        copy_calibration(args.copy_mb)
    names = workloads.ORDER if args.all else [args.workload]
    results = {n: measure(n, args.steps, args.warmup, eager=args.eager, path=args.path, exchange=args.exchange)
               for n in names}
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
        "timing": "eager launches" if args.eager else "HIP graph replays",
        "config": {"workload": args.workload, "form": main_res["form"], "B": main_res["B"], "E": main_res["E"], "topk": main_res["topk"],
                   "D": main_res["D"], "I": main_res["I"], "parallelism": "single GPU (one TP shard)"},
        "routes_per_s": round(main_res["routes_per_s"], 1),
        "hbm_gbs_unique_weights": round(main_res["step_gbs"], 1),
        "hbm_frac_of_peak": round(main_res["step_gbs"] / HBM_PEAK_GBS, 4),
        "roofline": {
            "bound": "hbm",
            "kernel": main_res["kernel"],
            "achieved": round(main_res["experts_gbs"], 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(main_res["experts_gbs"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(args.workload),
            "avg_us": round(main_res["experts_us"], 3),
            "alg_bytes": main_res["experts_alg_bytes"],
        },
        "cpu_baseline": cpu,
        "combine": {"kernel": "combine_kernel", "us": round(main_res["combine_us"], 3),
                    "alg_bytes": main_res["combine_alg_bytes"], "gbs": round(main_res["combine_gbs"], 1),
                    "note": "weighted top-k combine of the step's rows into [B, D]; not part of the step"},
    }
    if args.all:
        line["per_workload"] = {n: {"form": r["form"], "us": round(r["step_us"], 3),
                                    "experts_us": round(r["experts_us"], 3),
                                    "combine_us": round(r["combine_us"], 3),
                                    "routes_per_s": round(r["routes_per_s"], 1),
                                    "gbs_unique": round(r["step_gbs"], 1),
                                    "frac": round(r["step_gbs"] / HBM_PEAK_GBS, 4)} for n, r in results.items()}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
