#!/usr/bin/env python3
"""Benchmark of the fused pre-norm dilated Conv1d block on one MI355X.

One step = one call of prenorm_dconv1d_fwd on the N=32, C=256, L=4096, d=128 float32
workload: the BN fold + weight repack kernel and the fused implicit-GEMM kernel, with
all inputs resident in HBM. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense FP32 matrix peak
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_conv_f32_prenorm_N32_C256_L4096_d128.json")


def measured_traffic():
    """HBM bytes per launch of the dominant kernel from the committed PMC summary, or
    None when there is none or the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from normalisation_dilated_conv1d_amd.profiling import source_digest

    if t.get("source_sha256") != source_digest("conv_f32_kernel"):
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_baseline(w, min_seconds: float):
    """The float64 oracle, untuned, on the host cores: repeats the whole workload until
    at least `min_seconds` have passed (at least once)."""
    import numpy as np  # noqa: F401
    from threadpoolctl import threadpool_info

    import oracle
    from normalisation_dilated_conv1d_amd.inputs import prenorm_inputs, seed_for

    p = prenorm_inputs(w["N"], w["C"], w["L"], seed_for(1))
    flops = 2.0 * w["N"] * w["L"] * w["C"] * 3 * w["C"]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.prenorm_block(p["x"], p["running_mean"], p["running_var"], p["gamma"], p["beta"],
                             p["eps"], p["W"], p["b"], w["d"])
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    return {"value": round(flops * reps / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole N=32 C=256 L=4096 d=128 workload, float64 numpy oracle, "
                      f"{reps} run(s) in {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (PMC calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not "
              "supported (the block shards over the batch with no exchange, see the design "
              "notes)", file=sys.stderr)
        sys.exit(2)

    import torch

    import normalisation_dilated_conv1d_amd as dc
    from normalisation_dilated_conv1d_amd.inputs import WORKLOADS, prenorm_inputs, seed_for

    wl = WORKLOADS[1]
    w = wl.dims
    N, C, L, d = w["N"], w["C"], w["L"], w["d"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    p = prenorm_inputs(N, C, L, seed_for(1))
    q = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
    out = torch.empty_like(q["x"])

    def step():
        dc.prenorm_dconv1d_fwd(q["x"], q["running_mean"], q["running_var"], q["gamma"],
                               q["beta"], q["eps"], q["W"], q["b"], d, out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    total_ms = e0.elapsed_time(e1)
    ms_per_step = total_ms / args.steps

    # dominant kernel alone: HIP events recorded by the library around each launch of
    # the fused conv kernel, on the stream it is launched on
    with dc.KernelTimer() as kt:
        for _ in range(args.steps):
            step()
        kern_ms, launches = kt.read()
    kern_ms_avg = kern_ms / max(launches, 1)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    flops = 2.0 * N * L * C * 3 * C
    alg_bytes = 4.0 * (2 * N * C * L + 3 * C * C + 5 * C)
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    gbps = alg_bytes / (ms_per_step * 1e-3) / 1e9
    k_tflops = flops / (kern_ms_avg * 1e-3) / 1e12

    line = {
        "metric": "fused block TFLOP/s & GB/s (N32 C256 L4096 d128) vs MI355X roofline",
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": wl.name, "N": N, "C": C, "L": L, "kernel_size": 3,
                   "dilation": d, "padding": d, "parallelism": "single GPU"},
        "hbm_gbps_algorithmic": round(gbps, 2),
        "frac_fp32_mfma_peak": round(tflops / PEAK_FP32_MFMA_TFLOPS, 4),
        "roofline": {"bound": "mfma", "achieved": round(k_tflops, 3),
                     "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(k_tflops / PEAK_FP32_MFMA_TFLOPS, 4),
                     "traffic": measured_traffic(),
                     "kernel": "conv_f32_kernel<128, BN, residual, float>",
                     "kernel_ms": round(kern_ms_avg, 5),
                     "algorithmic_flops_per_launch": flops,
                     "algorithmic_bytes_per_launch": alg_bytes},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
