#!/usr/bin/env python3
"""Benchmark of the fused pre-norm dilated Conv1d block on one MI355X.

One step = one call of prenorm_dconv1d_fwd on the N=32, C=256, L=4096, d=128 float32
workload: the BN fold + weight repack kernel and the fused implicit-GEMM kernel, with
all inputs resident in HBM. Prints one JSON line.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-cpu-baseline]
                    [--no-other-workloads] [--workload 1|2|3|4] [--dilation D]

The default run (workload 1) also times the other workloads after the headline one and
adds them to the same line under "other_workloads": the dilation sweep (d = 1, 8, 512,
2048), Conv1d+GroupNorm and the bf16-storage block, each with its step time, its
dominant kernel's HIP-event time and that kernel's roofline fractions.
--workload 2 (the same block at dilation D, one of 1, 8, 512, 2048), 3 (Conv1d+GroupNorm)
and 4 (bf16 storage) time one of them alone, as the headline; the default, workload 1, is
the reported metric. For the block workloads,
--bn train times the training-mode entry point (batch-statistics pass, running-stat
update, then the same conv) and --bn external the entry point that takes an already
normalised input and a separate residual.
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
PEAK_BF16_MFMA_TFLOPS = 2500.0  # MI355X dense BF16 matrix peak
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
# committed PMC traffic records of the dominant kernel, per workload (eval-mode BN for the
# block workloads)
TRAFFIC_FILES = {
    1: ("conv_wino_kernel", os.path.join(ROOT, "profiles",
                                         "traffic_conv_wino_prenorm_N32_C256_L4096_d128.json")),
    4: ("conv_bf16_kernel", os.path.join(ROOT, "profiles",
                                         "traffic_conv_bf16_prenorm_N16_C512_L16384_d128.json")),
    3: ("conv_gn_fused_kernel",
        os.path.join(ROOT, "profiles", "traffic_conv_gn_fused_N16_Cin128_Cout256_T1024_G32.json")),
}


def measured_traffic(workload):
    """HBM bytes per launch of the dominant kernel from the committed PMC summary, or
    None when there is none or the kernel source changed since it was taken."""
    if workload not in TRAFFIC_FILES:
        return None
    kernel, path = TRAFFIC_FILES[workload]
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    from normalisation_dilated_conv1d_amd.profiling import source_digest

    if t.get("kernel") != kernel or t.get("source_sha256") != source_digest(kernel):
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


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
    # cores = the BLAS threads the oracle's matrix products ran on
    info = threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] or [1])
    blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                             for i in info if i.get("user_api") == "blas"})) or "unknown"
    return {"value": round(flops * reps / el / 1e12, 6), "unit": "TFLOP/s", "cores": threads,
            "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"whole N=32 C=256 L=4096 d=128 workload, float64 numpy oracle, "
                      f"{reps} run(s) in {el:.1f} s",
            "cpu": cpu_model(), "blas": blas}


def _kernel_name(workload_kind, bf16, winograd=False):
    if workload_kind == "groupnorm":
        # per-wave windows, 16-byte loads, the conv's form
        return f"conv_gn_fused_kernel<1, 4, {'true' if winograd else 'false'}>"
    if bf16:
        return "conv_bf16_kernel<pair, 8 waves>"
    return ("conv_wino_kernel<4> (Winograd F(2,3), 256-channel tiles)" if winograd
            else "conv_f32_kernel<128, 4, BN, residual, float>")


def winograd_mfma_flops(N, C, L, d, co_tile=256):
    """Multiply-add work the Winograd kernel runs on the matrix cores for a float32 block:
    four GEMMs over (output channels padded to the channel tile: 256 for the benchmark's
    C = 256 and 512) x (input channels padded to 32) x (output pairs, in tiles of 32), two
    flops per multiply-add."""
    d = min(d, L)
    pairs = d * (L // (2 * d)) + min(d, L % (2 * d))     # pairs with an output in range
    pairs_run = -(-pairs // 32) * 32
    return 8.0 * N * (-(-C // co_tile) * co_tile) * (-(-C // 32) * 32) * pairs_run


def groupnorm_winograd_mfma_flops(N, C_in, C_out, T_out):
    """Multiply-add work the single-kernel Conv1d + GroupNorm path runs on the matrix cores
    in its Winograd form: per (sample, 16 output channels), ceil(T_out / 128) waves of 64
    output pairs, each four 16 x 16 x 4 MFMAs per pair block and K-step, four K-steps per
    16 input channels, two flops per multiply-add."""
    waves = -(-T_out // 128)
    return 2.0 * N * C_out * waves * 64 * 4 * C_in


def setup(workload, dilation, bn, dev):
    """Inputs resident on the device and the step of one workload: returns a dict with the
    step function, its algorithmic flops and bytes, the config and the dtype."""
    import torch

    import normalisation_dilated_conv1d_amd as dc
    from normalisation_dilated_conv1d_amd.inputs import (WORKLOADS, groupnorm_inputs,
                                                          prenorm_inputs, seed_for)

    wl = WORKLOADS[workload]
    w = wl.dims
    wname = wl.name if workload != 2 else f"{wl.name}_d{dilation}"
    if wl.kind == "prenorm":
        if workload == 2:
            w = dict(w, d=dilation)
        N, C, L, d = w["N"], w["C"], w["L"], w["d"]
        bf16 = w["dtype"] == "bf16"
        # the sweep's inputs are drawn per dilation, as in its parity tests
        p = prenorm_inputs(N, C, L, seed_for(workload, d if workload == 2 else 0), bf16=bf16)
        q = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
        out = torch.empty_like(q["x"])
        if bn == "eval":
            fn = dc.prenorm_dconv1d_fwd_bf16 if bf16 else dc.prenorm_dconv1d_fwd

            def step():
                fn(q["x"], q["running_mean"], q["running_var"], q["gamma"], q["beta"], q["eps"],
                   q["W"], q["b"], d, out=out)
        elif bn == "train":
            fn = dc.prenorm_dconv1d_fwd_train_bf16 if bf16 else dc.prenorm_dconv1d_fwd_train
            rm, rv = q["running_mean"].clone(), q["running_var"].clone()
            sm, si = torch.empty_like(rm), torch.empty_like(rm)

            def step():
                fn(q["x"], rm, rv, q["gamma"], q["beta"], q["eps"], 0.1, q["W"], q["b"], d,
                   out=out, save_mean=sm, save_invstd=si)
        else:
            fn = dc.relu_dconv1d_residual_fwd_bf16 if bf16 else dc.relu_dconv1d_residual_fwd
            # the caller's normalised activation, made once outside the timed region
            xn = torch.nn.functional.batch_norm(
                q["x"].float(), q["running_mean"], q["running_var"], q["gamma"], q["beta"],
                training=False, eps=q["eps"]).to(q["x"].dtype).contiguous()

            def step():
                fn(xn, q["W"], q["b"], q["x"], d, out=out)

        esz = 2 if bf16 else 4
        flops = 2.0 * N * L * C * 3 * C
        winograd = (not bf16) and dc.dconv1d_block_method(N, C, L, d) == dc.DCONV1D_METHOD_WINOGRAD
        mfma_flops = winograd_mfma_flops(N, C, L, d) if winograd else flops
        alg_bytes = esz * 2.0 * N * C * L + 4.0 * (3 * C * C + 5 * C)
        if bn != "eval":
            # train: the statistics pass reads x before the conv can start; external: the
            # normalised input and the residual are separate tensors
            alg_bytes += esz * 1.0 * N * C * L
        config = {"workload": wname, "N": N, "C": C, "L": L, "kernel_size": 3,
                  "dilation": d, "padding": d, "bn_mode": bn, "parallelism": "single GPU",
                  "conv_method": "winograd_f2_3" if winograd else "direct_3tap"}
        if workload == 2:
            # share of the counted (output step, tap) pairs whose input lies inside [0, L);
            # the metric counts the padded ones too
            config["valid_tap_share"] = round((L + 2 * max(L - d, 0)) / (3 * L), 4)
    else:
        N, C_in, C_out, T, G = w["N"], w["C_in"], w["C_out"], w["T"], w["G"]
        p = groupnorm_inputs(N, C_in, C_out, T, seed_for(workload))
        q = {k: (v.to(dev) if isinstance(v, torch.Tensor) else v) for k, v in p.items()}
        T_out = T + 2 * w["padding"] - 2 * w["dilation"]
        out = torch.empty((N, C_out, T_out), device=dev)
        bf16 = False

        def step():
            dc.conv1d_groupnorm_fwd(q["x"], q["W"], q["bias"], q["gamma"], q["beta"], q["eps"],
                                    G, w["padding"], w["dilation"], out=out)

        flops = 2.0 * N * T_out * C_out * 3 * C_in
        winograd = dc.dconv1d_groupnorm_method(N, C_in, C_out, T, G, w["padding"], w["dilation"],
                                               x=q["x"], W=q["W"]) == dc.DCONV1D_METHOD_WINOGRAD
        mfma_flops = groupnorm_winograd_mfma_flops(N, C_in, C_out, T_out) if winograd else flops
        # one launch (every group inside one workgroup): x once, out written once, W and
        # the affine vectors; the conv output never reaches HBM
        alg_bytes = 4.0 * (N * C_in * T + N * C_out * T_out + 3 * C_in * C_out + 2 * C_out)
        config = {"workload": wl.name, "N": N, "C_in": C_in, "C_out": C_out, "T": T,
                  "num_groups": G, "kernel_size": 3, "padding": w["padding"],
                  "dilation": w["dilation"], "parallelism": "single GPU",
                  "conv_method": "winograd_f2_3" if winograd else "direct_3tap"}
    return {"step": step, "flops": flops, "mfma_flops": mfma_flops, "alg_bytes": alg_bytes,
            "config": config, "bf16": bf16, "kernel": _kernel_name(wl.kind, bf16, winograd),
            "out": out}


def timed(step, steps, warmup, dev, warmup_ms=0.0):
    """Mean ms per step over `steps` steps after `warmup` untimed ones (HIP events on the
    current stream), and the mean duration of the dominant kernel over another `steps`
    steps (HIP events the library records around each launch, on its stream). With
    warmup_ms, more untimed steps follow the `warmup` ones until about that much GPU time
    has passed (the GPU's clocks fall while the host prepares a workload's inputs)."""
    import torch

    import normalisation_dilated_conv1d_amd as dc

    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    if warmup_ms > 0:
        per = (time.perf_counter() - t0) * 1e3 / max(warmup, 1)
        for _ in range(int(warmup_ms / max(per, 1e-3))):
            step()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / steps
    with dc.KernelTimer() as kt:
        for _ in range(steps):
            step()
        kern_ms, launches = kt.read()
    return ms_per_step, kern_ms / max(launches, 1)


def roofline(flops, alg_bytes, kern_ms, bf16, traffic, mfma_flops=None):
    """Roofline record of the dominant kernel: MFMA-bound, with the HBM side reported
    against 8 TB/s from the algorithmic bytes and (when a current counter record exists)
    the measured traffic. `achieved` and `frac` count the direct conv's nominal flops
    (2*N*L*C_out*3*C_in); the Winograd kernel runs 2/3 of them on the matrix cores, so
    `mfma_executed_frac` is its use of the matrix cores and `frac` may exceed it."""
    peak = PEAK_BF16_MFMA_TFLOPS if bf16 else PEAK_FP32_MFMA_TFLOPS
    mfma_flops = flops if mfma_flops is None else mfma_flops
    k_tflops = flops / (kern_ms * 1e-3) / 1e12
    x_tflops = mfma_flops / (kern_ms * 1e-3) / 1e12
    alg_gbps = alg_bytes / (kern_ms * 1e-3) / 1e9
    rec = {"bound": "mfma", "achieved": round(k_tflops, 3), "peak": peak, "unit": "TFLOP/s",
           "frac": round(k_tflops / peak, 4), "traffic": traffic,
           "kernel_ms": round(kern_ms, 5),
           "mfma_executed_flops_per_launch": mfma_flops,
           "mfma_executed_tflops": round(x_tflops, 3),
           "mfma_executed_frac": round(x_tflops / peak, 4),
           "algorithmic_flops_per_launch": flops, "algorithmic_bytes_per_launch": alg_bytes,
           "hbm_gbps_algorithmic": round(alg_gbps, 2),
           "hbm_frac_algorithmic": round(alg_gbps / PEAK_HBM_GBPS, 4)}
    if traffic is not None:
        t_gbps = traffic / (kern_ms * 1e-3) / 1e9
        rec["hbm_gbps_traffic"] = round(t_gbps, 2)
        rec["hbm_frac_traffic"] = round(t_gbps / PEAK_HBM_GBPS, 4)
    return rec


def other_workloads(dev, steps, warmup):
    """The dilation sweep, Conv1d+GroupNorm and the bf16 block, each timed like the
    headline workload (mean ms per step, the dominant kernel's HIP-event time and its
    roofline fraction); parity for all of them is checked by the GPU tests."""
    res = {}
    for workload, dil in ((2, 1), (2, 8), (2, 512), (2, 2048), (3, None), (4, None)):
        s = setup(workload, dil, "eval", dev)
        ms, kms = timed(s["step"], steps, warmup, dev, warmup_ms=100.0)
        rec = roofline(s["flops"], s["alg_bytes"], kms, s["bf16"], measured_traffic(workload),
                       s["mfma_flops"])
        rec["kernel"] = s["kernel"]
        res[s["config"]["workload"]] = {
            "ms_per_step": round(ms, 5), "kernel_ms": round(kms, 5),
            "value": round(s["flops"] / (ms * 1e-3) / 1e12, 3), "unit": "TFLOP/s",
            "dtype": "bf16" if s["bf16"] else "f32", "config": s["config"], "roofline": rec}
        del s
    return res


# The pages' own figures for this workload are back-of-envelope estimates of memory
# traffic on a roughly 900 GB/s GPU, not measurements (pre-norm block page, design turn).
PAGE_ESTIMATES = {"note": "page estimate, not measured",
                  "unfused_traffic_bytes": 1.2e9, "fused_traffic_bytes": 2.7e8}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="time only the selected workload (the default run also times the "
                         "dilation sweep, Conv1d+GroupNorm and the bf16 block)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (PMC calibration)")
    ap.add_argument("--workload", type=int, default=1, choices=(1, 2, 3, 4),
                    help="1: fp32 block N32 C256 L4096 d128 (default, the reported metric); "
                         "2: the same block at --dilation D (1, 8, 512 or 2048); "
                         "3: Conv1d+GroupNorm N16 Cin128 Cout256 T1024 G32; "
                         "4: bf16-storage block N16 C512 L16384 d128")
    ap.add_argument("--dilation", type=int, default=None,
                    help="workload 2: the dilation (= padding) of the sweep to time")
    ap.add_argument("--bn", default="eval", choices=("eval", "train", "external"),
                    help="block workloads: BatchNorm in eval mode (default), training mode, "
                         "or done by the caller (ReLU + conv + separate residual)")
    args = ap.parse_args()

    if args.bn != "eval" and args.workload == 3:
        ap.error("--bn applies to the block workloads (1, 2 and 4)")
    if (args.dilation is not None) != (args.workload == 2):
        ap.error("--dilation goes with --workload 2, and workload 2 needs it")
    if args.gpus != 1:
        print(f"bench.py: measures one GPU only; --gpus {args.gpus} is not supported (the "
              "block would shard over the batch with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from normalisation_dilated_conv1d_amd.inputs import WORKLOADS

    if args.workload == 2 and args.dilation not in WORKLOADS[2].dims["ds"]:
        ap.error(f"--dilation must be one of {WORKLOADS[2].dims['ds']}")
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    s = setup(args.workload, args.dilation, args.bn, dev)
    step, flops, alg_bytes, bf16 = s["step"], s["flops"], s["alg_bytes"], s["bf16"]
    config = s["config"]
    wname = config["workload"]

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

    # per-step durations (median), warm and with the MALL flushed: before each cold step a
    # 512 MiB scratch buffer is overwritten ("write"), so x (134 MB for the default
    # workload) does not stay resident in the 256 MB last-level cache between steps, and
    # the caches hold the scratch's dirty lines, written back while the step runs; or it
    # is read ("read": summed), which also evicts x but leaves nothing to write back
    # The flushed passes also return the conv kernel's mean duration over their steps (the
    # library's event pair around each launch; the warm pass runs without it, as the pair
    # adds a little to each step).
    def per_step_ms(flush):
        import contextlib

        import normalisation_dilated_conv1d_amd as dc

        scratch = torch.ones(512 * (1 << 20) // 4, device=dev) if flush else None
        sink = torch.empty((), device=dev)
        times = []
        with (dc.KernelTimer() if flush else contextlib.nullcontext()) as kt:
            for i in range(args.steps):
                if flush == "write":
                    scratch.fill_(float(i))
                elif flush == "read":
                    torch.sum(scratch, dim=0, out=sink)
                a_ev = torch.cuda.Event(enable_timing=True)
                b_ev = torch.cuda.Event(enable_timing=True)
                a_ev.record(stream)
                step()
                b_ev.record(stream)
                times.append((a_ev, b_ev))
            torch.cuda.synchronize()
            k_ms, k_n = kt.read() if flush else (0.0, 0)
        ms = sorted(a_ev.elapsed_time(b_ev) for a_ev, b_ev in times)
        del scratch
        return ms[len(ms) // 2], k_ms / max(k_n, 1)

    warm_median, _ = per_step_ms(None)
    cold_median, cold_kern = per_step_ms("write")
    cold_read_median, cold_read_kern = per_step_ms("read")

    # dominant kernel alone: HIP events recorded by the library around each launch of
    # the fused conv kernel, on the stream it is launched on
    import normalisation_dilated_conv1d_amd as dc

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

    peak = PEAK_BF16_MFMA_TFLOPS if bf16 else PEAK_FP32_MFMA_TFLOPS
    tflops = flops / (ms_per_step * 1e-3) / 1e12
    gbps = alg_bytes / (ms_per_step * 1e-3) / 1e9
    metric = ("fused block TFLOP/s & GB/s (N32 C256 L4096 d128) vs MI355X roofline"
              if args.workload == 1 and args.bn == "eval"
              else f"TFLOP/s & GB/s, {wname}, BN {args.bn}, vs MI355X roofline"
              if "C" in config else f"TFLOP/s & GB/s, {wname}, vs MI355X roofline")
    rl = roofline(flops, alg_bytes, kern_ms_avg, bf16,
                  measured_traffic(args.workload) if args.bn == "eval" else None,
                  s["mfma_flops"])
    rl["kernel"] = s["kernel"]

    line = {
        "metric": metric,
        "value": round(tflops, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic",
        "config": config,
        "hbm_gbps_algorithmic": round(gbps, 2),
        "ms_per_step_median": round(warm_median, 5),
        "ms_per_step_median_cold_mall": round(cold_median, 5),
        "ms_per_step_median_cold_mall_read": round(cold_read_median, 5),
        "kernel_ms_cold_mall": round(cold_kern, 5),
        "kernel_ms_cold_mall_read": round(cold_read_kern, 5),
        "frac_mfma_peak": round(tflops / peak, 4),
        "roofline": rl,
    }
    del s, step
    if args.workload == 1 and args.bn == "eval":
        line["page_traffic_estimates"] = PAGE_ESTIMATES
        if not args.no_other_workloads:
            line["other_workloads"] = other_workloads(dev, min(args.steps, 30),
                                                      min(args.warmup, 20))
        if not args.no_cpu_baseline:
            line["cpu_baseline"] = cpu_baseline(WORKLOADS[1].dims, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
