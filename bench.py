#!/usr/bin/env python3
"""Benchmark of the routed-experts MoE decode step on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input: the MXFP8
plan of x, the unit table and the persistent experts kernel (FC1 -> SwiGLU -> hidden
requant -> FC2 -> BF16 rows).  For B <= 8 that is one moe_decode_run launch (the
kernel quantizes and routes the batch itself); for larger batches two calls,
moe_plan_group (the plan of x and the unit table) + moe_experts_run.  Inputs are
resident in HBM before the timed region starts.  Step i reads replica i % R of the
weights, with R * (weight bytes a step touches) >= 1 GiB, so the 256 MB Infinity Cache
cannot serve a weight byte twice.  The steps are captured in one HIP graph
(torch.cuda.CUDAGraph) and replayed; the timed region is bracketed by synchronizations
and HIP events on the launch stream.

By default all five workloads are timed.  Prints ONE JSON line: `value` is µs per layer
of the headline workload (wide_b256, B = 256, the largest the metric names; --workload
picks another), `roofline` is its dominant kernel (algorithmic bytes / the kernel's
average duration, HIP events over graph replays of that kernel alone), `cpu_baseline`
the oracle on the host cores (best of 3), and `per_workload` the same figures for
every workload, with the oracle also on one thread for the three smallest, and the
weighted top-k combine (moe_combine) of the step's rows timed alone (it follows the
step; it is not part of it).
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "kernel_traffic.json")


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


ROTATE_BYTES = 1 << 30  # bytes a step sequence touches before it reads a replica again


def measure(d: dict, steps: int, warmup: int, *, eager: bool = False, path: str = "auto",
            exchange: int | None = None, log=print) -> dict:
    """Times `steps` steps of workload d on the GPU (inputs resident in HBM).  Step i reads
    replica i % R of the expert weights, R = ceil(1 GiB / weight bytes a step touches),
    so no weight byte is read again before 1 GiB of others: the 256 MB Infinity Cache
    cannot serve it."""
    import numpy as np
    import torch

    from moe_routed_expert_mx_amd.layer import MoeLayer

    w = d["workload"]
    uniq = _unique_weight_bytes(d["ids"], w)
    R = max(2, math.ceil(ROTATE_BYTES / uniq))
    layer = MoeLayer(d["w13"], d["s13"], d["w2"], d["s2"], B_max=w.B, topk=w.K, device="cuda", replicas=R)
    x = torch.from_numpy(d["x"]).cuda()
    ids = torch.from_numpy(d["ids"]).cuda()
    rw = torch.from_numpy(d["weights"]).cuda()
    out = layer.out_buffer(w.B)
    y = torch.empty(w.B, w.D, dtype=torch.bfloat16, device="cuda")
    decode = w.B <= MoeLayer.DECODE_MAX and (path == "decode" or (path == "auto" and MoeLayer.AUTO_DECODE))
    form = "decode" if decode else "grouped"
    xo = {"exchange": exchange} if (decode and exchange is not None) else {}

    for i in range(warmup):
        layer.forward(x, ids, out, replica=i % R, path=form, **xo)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()

    def step(i):
        layer.forward(x, ids, out, replica=i % R, path=form, **xo)

    def kernel(i):  # the dominant kernel alone (the decode form's step is that kernel)
        if decode:
            step(i)
        else:
            layer.experts(w.B, out, replica=i % R)

    def comb(i):
        layer.combine(out, rw, y)

    def one_launch(i):  # B > 8: the whole step as one launch (plan and chunk table inside it)
        layer.forward(x, ids, out, replica=i % R, path="decode")

    seqs = [("step", step), ("kernel", kernel), ("combine", comb)]
    if not decode:
        seqs.append(("one_launch", one_launch))

    graphs = {}
    if not eager:
        # one graph of all `steps` steps for each timed sequence: exactly `steps` steps
        # are timed, each on its own replica
        for key, fn in seqs:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(steps):
                    fn(i)
            graphs[key] = g
        for g in graphs.values():
            g.replay()
        layer.forward(x, ids, out, path=form, **xo)  # plan and units of this batch for the kernel-only graph
        torch.cuda.synchronize()

    def timed(key, fn) -> float:
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        if eager:
            for i in range(steps):
                fn(i)
        else:
            graphs[key].replay()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) * 1e3 / steps

    step_us = timed("step", step)
    kernel_us = timed("kernel", kernel)
    combine_us = timed("combine", comb)
    one_launch_us = timed("one_launch", one_launch) if not decode else None
    combine_bytes = w.B * w.K * w.D * 2 + w.B * w.K * 4 + w.B * w.D * 2  # rows, weights, y

    io_bytes = w.B * w.D * 2 + w.B * w.K * 4 + w.B * w.K * w.D * 2  # x, ids, out
    plan_bytes = w.B * w.D * 33 // 32
    # weights + the activations the kernel reads (the plan, or x and ids in the decode
    # form) + output rows
    act_bytes = w.B * w.D * 2 + w.B * w.K * 4 if decode else plan_bytes
    kernel_bytes = uniq + act_bytes + w.B * w.K * w.D * 2
    res = {
        "workload": w.name, "form": form, "kernel": layer.kernel_name(w.B, path=form, **xo),
        "B": w.B, "E": w.E, "topk": w.K, "D": w.D, "I": w.I,
        "distinct_experts": int(len(np.unique(d["ids"]))), "replicas": R, "rotated_bytes": R * uniq,
        "step_us": step_us, "kernel_us": kernel_us,
        "routes_per_s": w.B * w.K / (step_us * 1e-6),
        "unique_weight_bytes": uniq, "step_bytes": uniq + io_bytes,
        "kernel_alg_bytes": kernel_bytes,
        "step_gbs": uniq / (step_us * 1e-6) / 1e9,
        "kernel_gbs": kernel_bytes / (kernel_us * 1e-6) / 1e9,
        "flops": 6 * w.I * w.D * w.B * w.K,
        "combine_us": combine_us, "combine_alg_bytes": combine_bytes,
        "one_launch_step_us": one_launch_us,
        "combine_gbs": combine_bytes / (combine_us * 1e-6) / 1e9,
    }
    log(json.dumps({"config_detail": res}), file=sys.stderr)
    del graphs, layer
    torch.cuda.empty_cache()
    return res


def cpu_baseline(d: dict, threads: int, max_routes: int | None, repeats: int = 3) -> dict:
    """The oracle (plan + per-route FC1/SwiGLU/requant/FC2 in FP64) on `threads` host
    threads, best of `repeats` runs, on the whole layer or a seeded sample of at most
    `max_routes` routes (then scaled to the layer by route count: routes are independent
    and cost the same)."""
    import numpy as np

    import oracle

    w = d["workload"]
    R = w.B * w.K
    routes = None
    if max_routes is not None and R > max_routes:
        routes = np.random.default_rng(0).choice(R, max_routes, replace=False).astype(np.int32)
    n_routes = R if routes is None else len(routes)
    best = float("inf")
    for _ in range(repeats):
        t0 = time.perf_counter()
        codes, scales = oracle.plan(d["x"])
        oracle.experts(d["w13"], d["s13"], d["w2"], d["s2"], codes, scales, d["ids"],
                       hidden_floor=oracle.default_hidden_floor(w.I), routes=routes, nthreads=threads,
                       want_hidden=False)
        best = min(best, time.perf_counter() - t0)
    layer_us = best / n_routes * R * 1e6
    sample = (f"best of {repeats} oracle runs (plan + {n_routes} of {R} routes, "
              f"{'all' if routes is None else 'a seeded random sample'}) on {threads} thread(s): "
              f"{best:.3f} s, scaled to the layer")
    return {"value": layer_us, "unit": "us", "cores": threads, "kind": "oracle", "sample": sample}


def kernel_roofline(r: dict) -> dict:
    return {
        "bound": "hbm",
        "kernel": r["kernel"],
        "achieved": round(r["kernel_gbs"], 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(r["kernel_gbs"] / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(r["workload"]),
        "avg_us": round(r["kernel_us"], 3),
        "alg_bytes": r["kernel_alg_bytes"],
    }


HEADLINE = "wide_b256"  # the largest configuration the metric names (B = 256)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=None,
                    help="time only this workload (default: all five; the headline is wide_b256)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
    names = [args.workload] if args.workload else list(workloads.ORDER)
    head = args.workload or HEADLINE
    threads = max(1, len(os.sched_getaffinity(0)))
    results, cpu = {}, {}
    for n in names:
        d = workloads.generate(n)
        print(f"bench: {n}", file=sys.stderr, flush=True)
        results[n] = measure(d, args.steps, args.warmup, eager=args.eager, path=args.path, exchange=args.exchange)
        if not args.no_cpu_baseline:
            big = d["workload"].B * d["workload"].K > 256
            cpu[n] = {"threads": cpu_baseline(d, threads, 512 if big else None)}
            if n in ("tiny", "decode_b1", "decode_b8"):
                cpu[n]["one_thread"] = cpu_baseline(d, 1, None)
        del d
    main_res = results[head]
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
        "timing": "eager launches" if args.eager else "HIP graph replays, one replica per step (cold)",
        "config": {"workload": head, "form": main_res["form"], "B": main_res["B"], "E": main_res["E"],
                   "topk": main_res["topk"], "D": main_res["D"], "I": main_res["I"],
                   "parallelism": "single GPU (one TP shard)"},
        "routes_per_s": round(main_res["routes_per_s"], 1),
        "hbm_gbs_unique_weights": round(main_res["step_gbs"], 1),
        "hbm_frac_of_peak": round(main_res["step_gbs"] / HBM_PEAK_GBS, 4),
        "roofline": kernel_roofline(main_res),
        "cpu_baseline": cpu.get(head, {}).get("threads"),
        "per_workload": {},
    }
    for n, r in results.items():
        line["per_workload"][n] = {
            "form": r["form"], "us": round(r["step_us"], 3), "routes_per_s": round(r["routes_per_s"], 1),
            "gbs_unique": round(r["step_gbs"], 1), "frac": round(r["step_gbs"] / HBM_PEAK_GBS, 4),
            "distinct_experts": r["distinct_experts"], "replicas": r["replicas"],
            "rotated_bytes": r["rotated_bytes"], "tflops": round(r["flops"] / (r["step_us"] * 1e-6) / 1e12, 2),
            "roofline": kernel_roofline(r),
            "combine": {"kernel": "combine_kernel", "us": round(r["combine_us"], 3),
                        "alg_bytes": r["combine_alg_bytes"], "gbs": round(r["combine_gbs"], 1),
                        "note": "weighted top-k combine of the step's rows into [B, D]; not part of the step"},
            "cpu_baseline": {k: {"us": round(v["value"], 1), "cores": v["cores"], "sample": v["sample"]}
                             for k, v in cpu.get(n, {}).items()},
        }
        if r["one_launch_step_us"] is not None:
            line["per_workload"][n]["one_launch"] = {
                "kernel": "grouped_kernel (one launch)", "us": round(r["one_launch_step_us"], 3),
                "note": "the step as one moe_decode_run launch (plan and chunk table inside the grouped "
                        "kernel); the default step is moe_plan_group + moe_experts_run"}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
