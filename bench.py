#!/usr/bin/env python3
"""Benchmark of the fused fp32 linear layer + tail on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one lin_epi_run (the whole hot path: GEMM + fused tail, plus the
second pass where the variant has one) over inputs already resident in HBM.
The default workload is 2048x8192x8192 with tail (a) (scale 0.5, Hardtanh
[-2, 2], exact-erf GELU).  W untimed warm-up steps, then exactly K timed
steps on the handle's stream, bracketed by device synchronisation.  Prints
one JSON line.

The "roofline" object times the dominant (GEMM) kernel with HIP events the
library records around each launch on its own stream, over K more steps run
right after the timed ones (the event records would add a few microseconds
per launch to the timed steps).  The "cpu_baseline" object times the CPU oracle (as it is, unmodified)
on a bounded sample of rows of the same workload, on this host's cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

METRIC = "fused linear+epilogue TFLOP/s and % fp32 MFMA peak, 2048×8192×8192"
PEAK_FP32_MFMA_TFLOPS = 157.3  # MI355X dense fp32 matrix peak (256 CU x 2.4 GHz x 256 FLOP/clk)
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "dense_linear_layer_amd", "csrc", f) for f in
                  ("gemm_mfma.hpp", "gemv_mfma.hpp", "epilogue.hpp", "dma_layout.hpp", "schedule.hpp", "lin_epi.hip")]


def kernel_source_hash() -> str:
    """Hash of the kernel sources with comments and blank space removed, so a
    comment-only edit does not invalidate counters taken on the same code."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        text = re.sub(r"//[^\n]*", "", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, tail: str, variant: str):
    """HBM bytes per launch of the main kernel from the committed rocprofv3
    counter runs (keyed "workload:tail:variant"), or None when they were
    taken on different kernel sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    entry = t.get("%s:%s:%s" % (workload, tail, variant))
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("hbm_bytes_per_launch")


def cpu_baseline(w: workloads.Workload, X, W, b, target_s: float):
    """Time the oracle (linear + tail, unfused, fp64) on a bounded row sample."""
    import oracle

    tail = w.tails[0]
    rows_all = np.random.default_rng(w.seed + 2).permutation(w.M).astype(np.int64)
    probe = rows_all[: min(8, w.M)]
    t0 = time.perf_counter()
    oracle.forward_rows(X, W, b, tail.kind, probe, **tail.params())
    t_probe = time.perf_counter() - t0
    n = int(max(8, min(w.M, round(len(probe) * target_s / max(t_probe, 1e-6)))))
    rows = rows_all[:n]
    t0 = time.perf_counter()
    oracle.forward_rows(X, W, b, tail.kind, rows, **tail.params())
    dt = time.perf_counter() - t0
    flops = 2.0 * n * w.N * w.K
    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": "%d of %d rows (all %d columns, full K=%d), fp64 naive loops + unfused tail %s; %.2f s; "
                  "full-problem time extrapolated %.1f s" % (n, w.M, w.N, w.K, tail.name, dt, dt * w.M / n),
    }


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="p1_2048x8192x8192", choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--tail", type=int, default=None, help="tail index within the workload (default 0)")
    ap.add_argument("--split-k", type=int, default=0, help="0 auto, 1 off, S>=2 forced")
    ap.add_argument("--tile", type=int, default=0, help="0 auto, else a tile configuration (LIN_EPI_OPT_TILE)")
    ap.add_argument("--grid", type=int, default=0, help="0 auto, else a forced GEMM grid (LIN_EPI_OPT_GRID)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--reg-staging", action="store_true",
                    help="ablation: stage operand tiles through registers instead of direct-to-LDS loads")
    ap.add_argument("--unfused", action="store_true",
                    help="time the unfused ablation (GEMM to memory, then a separate tail kernel)")
    ap.add_argument("--pool-fold", action="store_true",
                    help="tail (b) via window-averaged weights: the GEMM is M x N/16 x K (FLOPs counted as such)")
    ap.add_argument("--scale-fold", action="store_true",
                    help="tail (a) with its scale folded into W and b (scale 1 in the epilogue)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 256 MiB device copy (reference kernel for HBM counter scaling)")
    args = ap.parse_args()

    if args.gpus != 1:
        print("bench.py runs on one GPU only: the library has no multi-GPU path (requested --gpus %d)" % args.gpus,
              file=sys.stderr)
        return 2
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py is single-process; WORLD_SIZE=%s is not supported" % os.environ["WORLD_SIZE"],
              file=sys.stderr)
        return 2

    import torch

    import dense_linear_layer_amd as lib

    w = workloads.WORKLOADS[args.workload]
    tail = w.tails[args.tail or 0]
    print("bench: %s %dx%dx%d tail %s" % (w.name, w.M, w.N, w.K, tail.name), file=sys.stderr, flush=True)
    X, W, b = workloads.make_inputs(w.M, w.N, w.K, seed=w.seed)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    with torch.cuda.stream(stream):
        Xd = torch.from_numpy(X).to(dev)
        Wd = torch.from_numpy(W).to(dev)
        bd = torch.from_numpy(b).to(dev)
        Y = torch.empty(lib.LinEpi.output_shape(w.M, w.N, tail.kind), dtype=torch.float32, device=dev)
    stream.synchronize()
    ref_tail = tail
    h = lib.LinEpi(stream=stream)
    h.set_option(lib.LIN_EPI_OPT_SPLIT_K, args.split_k)
    h.set_option(lib.LIN_EPI_OPT_TILE, args.tile)
    h.set_option(lib.LIN_EPI_OPT_GRID, args.grid)
    h.set_option(lib.LIN_EPI_OPT_UNFUSED, 1 if args.unfused else 0)
    h.set_option(lib.LIN_EPI_OPT_REG_STAGING, 1 if args.reg_staging else 0)
    flops = float(w.flops)
    prep_ms = None
    if args.pool_fold:
        if tail.kind != workloads.POOL_GELU_SCALE_ROWMAX:
            print("--pool-fold applies to tail (b) workloads only", file=sys.stderr)
            return 2
        # one-time preparation per weight, timed on its own
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            e0.record(stream)
            Wd_run, bd_run = h.pool_weights(Wd, bd, tail.pool_kernel)
            e1.record(stream)
        torch.cuda.synchronize()
        prep_ms = e0.elapsed_time(e1)
        tail = workloads.TAIL_B_FOLDED
        flops = 2.0 * w.M * (w.N // 16) * w.K
    elif args.scale_fold:
        if tail.kind != workloads.SCALE_HARDTANH_GELU:
            print("--scale-fold applies to tail (a) only (the other tails scale after a nonlinearity)",
                  file=sys.stderr)
            return 2
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(3):
            e0.record(stream)
            Wd_run, bd_run = h.scale_weights(Wd, bd, tail.scale)
            e1.record(stream)
        torch.cuda.synchronize()
        prep_ms = e0.elapsed_time(e1)
        tail = workloads.Tail(tail.kind, scale=1.0, lo=tail.lo, hi=tail.hi)
    else:
        Wd_run, bd_run = Wd, bd
    desc = lib.make_desc(tail.kind, tail.scale, tail.lo, tail.hi, tail.pool_kernel)

    # quick parity spot check of the benchmarked output (4 rows), before the
    # warm-up: the engine clock ramps up over ~25 ms of continuous load and
    # drops again when the device idles, so nothing may sit between the
    # warm-up and the timed steps
    import oracle

    h.run_into(Xd, Wd_run, bd_run, desc, Y)
    rows = workloads.checked_rows(w.M, seed=w.seed)[:4]
    ref = oracle.forward_rows(X, W, b, ref_tail.kind, rows, **ref_tail.params())
    got = Y.cpu().numpy().astype(np.float64)[rows]
    spot_err = float(np.max(np.abs(got - ref)))
    spot_ok = bool(np.all(np.abs(got - ref) <= 1e-3 * (1 + np.abs(ref))))

    # one event between consecutive steps: the per-step spread comes from the
    # same timed run as the total
    marks = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    for _ in range(args.warmup):
        h.run_into(Xd, Wd_run, bd_run, desc, Y)
    torch.cuda.synchronize()
    marks[0].record(stream)
    for i in range(args.steps):
        h.run_into(Xd, Wd_run, bd_run, desc, Y)
        marks[i + 1].record(stream)
    torch.cuda.synchronize()
    total_ms = marks[0].elapsed_time(marks[-1])
    step_times = sorted(marks[i].elapsed_time(marks[i + 1]) for i in range(args.steps))
    # per-kernel durations: the same K steps once more, right away (clock
    # still up), with the library's HIP events around every kernel on its
    # stream; kept out of the timed steps, where the extra event records add
    # 4-8 us per kernel launch to the step time
    h.profile()  # discard anything recorded so far
    h.set_option(lib.LIN_EPI_OPT_PROFILE, 1)
    for _ in range(args.steps):
        h.run_into(Xd, Wd_run, bd_run, desc, Y)
    prof = h.profile()
    h.set_option(lib.LIN_EPI_OPT_PROFILE, 0)
    plan = h.plan()

    if args.copy_calibration:
        src = torch.empty(64 * 1024 * 1024, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    ms_per_step = total_ms / args.steps
    value = flops / (ms_per_step * 1e-3) / 1e12
    gemm_ms = prof.total_ms[0] / max(1, prof.launches[0])
    variant = ("pool_fold" if args.pool_fold else "scale_fold" if args.scale_fold
               else "unfused" if args.unfused else "reg_staging" if args.reg_staging else "fused")
    traffic = measured_traffic(w.name, ref_tail.name, variant)
    # compulsory HBM bytes of one GEMM launch (X, W, b read once, the output
    # written once) over its duration: the weight-streaming figure, reported
    # for every workload beside whichever roofline bounds it
    if args.pool_fold:
        alg_bytes = 4.0 * (w.M * w.K + (w.N // 16) * (w.K + 1) + w.M)
    else:
        alg_bytes = float(w.algorithmic_bytes(tail))
    # plus the partial sums of split tiles, each written once and read once
    partial_bytes = 2.0 * plan.partial_bytes
    hbm_gbs = (alg_bytes + partial_bytes) / (gemm_ms * 1e-3) / 1e9
    hbm = {"achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
           "frac": round(hbm_gbs / PEAK_HBM_GBS, 4), "algorithmic_bytes": int(alg_bytes),
           "partial_bytes": int(partial_bytes)}
    if w.bound == "hbm":
        # weight-streaming regime: algorithmic bytes per launch / launch time
        alg_gbs = alg_bytes / (gemm_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(alg_gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(alg_gbs / PEAK_HBM_GBS, 4)}
    else:
        achieved = flops / (gemm_ms * 1e-3) / 1e12
        roofline = {"bound": "mfma", "achieved": round(achieved, 3), "peak": PEAK_FP32_MFMA_TFLOPS,
                    "unit": "TFLOP/s", "frac": round(achieved / PEAK_FP32_MFMA_TFLOPS, 4)}
    roofline.update({
        "traffic": traffic,
        "kernel_ms": round(gemm_ms, 5),
        "launches": int(prof.launches[0]),
        "second_pass_ms": round(prof.total_ms[1] / prof.launches[1], 5) if prof.launches[1] else None,
        "tail_pass_ms": round(prof.total_ms[2] / prof.launches[2], 5) if prof.launches[2] else None,
    })
    out = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "step_ms": {"median": round(float(np.median(step_times)), 5), "min": round(step_times[0], 5),
                    "max": round(step_times[-1], 5)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: X~N(0,1), W,b~U(+-1/sqrt(K)))",
        "config": {
            "workload": w.name,
            "M": w.M, "N": w.N, "K": w.K,
            "tail": tail.name,
            "tile": [plan.tile_m, plan.tile_n, plan.tile_k],
            "split_k": plan.split_k,
            "kernels_per_step": plan.kernels,
            "frac_of_fp32_mfma_peak": round(value / PEAK_FP32_MFMA_TFLOPS, 4),
            "variant": variant,
        },
        "roofline": roofline,
        "hbm": hbm,
        "parity_spot_check": {"rows": 4, "max_abs_err": spot_err, "ok": spot_ok},
    }
    if args.scale_fold:
        out["config"]["scale_weights_prep_ms"] = round(prep_ms, 5)
    if args.pool_fold:
        out["config"]["pool_weights_prep_ms"] = round(prep_ms, 5)
        out["config"]["gemm_flops_counted"] = "2*M*(N/16)*K"
        out["config"]["equivalent_unfolded_tflops"] = round(w.flops / (ms_per_step * 1e-3) / 1e12, 3)
    if not args.no_cpu_baseline:
        print("bench: timing the CPU oracle", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(w, X, W, b, args.cpu_seconds)
    h.close()
    print(json.dumps(out), flush=True)
    return 0 if spot_ok else 1


if __name__ == "__main__":
    sys.exit(main())
