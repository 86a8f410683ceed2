"""Summaries of rocprofv3 output for the library's kernels.

    python -m normalisation_dilated_conv1d_amd.profiling stats KERNEL_STATS_CSV --cmd "..."
        Markdown table of per-kernel call counts and durations from a
        ``rocprofv3 --kernel-trace --stats --output-format csv`` run.

    python -m normalisation_dilated_conv1d_amd.profiling warm KERNEL_TRACE_CSV --kernel NAME
        Average and median duration of one kernel's dispatches in a ``--kernel-trace`` run,
        leaving out the dispatches that follow one of bench.py's cache-flush kernels (a fill
        or a reduction over a scratch buffer; reported separately).

    python -m normalisation_dilated_conv1d_amd.profiling traffic \\
        --fetch FETCH_COUNTER_CSV --write WRITE_COUNTER_CSV --kernel conv_f32_kernel \\
        --calib-mib 192 --out profiles/traffic_....json --cmd-fetch "..." --cmd-write "..."
        HBM-side bytes per launch of one kernel from two ``rocprofv3 --pmc FETCH_SIZE`` /
        ``--pmc WRITE_SIZE`` runs. Both counters are scaled by what they read for a plain
        device-to-device copy of --calib-mib MiB in the same run (expected: that many MiB
        read and written), and the record carries the SHA-256 of the kernel's sources so a
        reader can tell when it no longer describes the current kernel.

    python -m normalisation_dilated_conv1d_amd.profiling mfma COUNTER_CSV --kernel conv_f32_kernel \
        --algorithmic-flops F --cmd "..."
        Executed MFMA work and MFMA-pipe utilisation per launch of one kernel from a
        ``rocprofv3 --pmc SQ_INSTS_VALU_MFMA_MOPS_<type> SQ_VALU_MFMA_BUSY_CYCLES
        GRBM_GUI_ACTIVE`` run: flops = MOPS * 512; utilisation = busy cycles /
        (per-XCD active cycles * SIMDs), where the reported GRBM_GUI_ACTIVE is the sum
        over the 8 XCDs and the part has 1024 SIMDs.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
KERNEL_SOURCES = {
    "conv_f32_kernel": ["normalisation_dilated_conv1d_amd/csrc/conv_f32.hip",
                        "normalisation_dilated_conv1d_amd/csrc/internal.h"],
    "conv_wino_kernel": ["normalisation_dilated_conv1d_amd/csrc/conv_wino.hip",
                         "normalisation_dilated_conv1d_amd/csrc/internal.h"],
    "conv_bf16_kernel": ["normalisation_dilated_conv1d_amd/csrc/conv_bf16.hip",
                         "normalisation_dilated_conv1d_amd/csrc/internal.h"],
    "conv_gn_fused_kernel": ["normalisation_dilated_conv1d_amd/csrc/conv_gn.hip",
                             "normalisation_dilated_conv1d_amd/csrc/conv_gn.h",
                             "normalisation_dilated_conv1d_amd/csrc/internal.h"],
}


def strip_comments(src: str) -> str:
    """C/C++ source without its comments, each whitespace run collapsed to one space:
    the code the compiler sees. String and character literals are kept as they are."""
    out = []
    i, n = 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def source_digest(kernel: str) -> str:
    """Digest of a kernel's sources with comments and layout ignored, plus any compile flags
    given to those files alone, so that a counter record stays valid across comment-only
    edits and goes stale on any change to the code or to how it is compiled."""
    from normalisation_dilated_conv1d_amd.build import FILE_FLAGS
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(strip_comments(f.read()).encode())
        extra = FILE_FLAGS.get(os.path.basename(rel))
        if extra:
            h.update(("\0flags:" + " ".join(extra)).encode())
    return h.hexdigest()


def _counter_rows(path):
    with open(path) as f:
        return list(csv.DictReader(f))


def stats_markdown(path: str, cmd: str) -> str:
    rows = list(csv.DictReader(open(path)))
    out = ["| kernel | calls | total (us) | average (us) | min (us) | max (us) | share |",
           "|---|---|---|---|---|---|---|"]
    for r in rows:
        name = r.get("Name") or r.get("KernelName") or r.get("Kernel_Name")
        calls = int(float(r.get("Calls", 0)))
        to_us = 1e-3  # rocprofv3 stats are in nanoseconds
        tot = float(r.get("TotalDurationNs", 0)) * to_us
        avg = float(r.get("AverageNs", 0)) * to_us
        mn = float(r.get("MinNs", 0)) * to_us
        mx = float(r.get("MaxNs", 0)) * to_us
        pct = float(r.get("Percentage", 0))
        out.append(f"| `{name[:90]}` | {calls} | {tot:.1f} | {avg:.2f} | {mn:.2f} | {mx:.2f} | {pct:.2f}% |")
    return "Command:\n\n```\n" + cmd + "\n```\n\n" + "\n".join(out) + "\n"


# kernels of bench.py's cold-cache passes: a scratch buffer overwritten (torch fill) or
# summed (torch reduction) before each such step
FLUSH_KERNELS = ("FillFunctor", "reduce_kernel")


def warm_split(trace_csv: str, kernel: str):
    """Durations (us) of the dispatches of `kernel` in a ``--kernel-trace`` CSV, split into
    warm ones and cold ones (those with a flush kernel, FLUSH_KERNELS, since the kernel's
    previous dispatch)."""
    rows = sorted(csv.DictReader(open(trace_csv)), key=lambda r: int(r["Start_Timestamp"]))
    warm, cold = [], []
    flushed = False
    for r in rows:
        name = r["Kernel_Name"]
        if any(f in name for f in FLUSH_KERNELS):
            flushed = True
        elif kernel in name:
            d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3
            (cold if flushed else warm).append(d)
            flushed = False
    return warm, cold


def warm_markdown(trace_csv: str, kernel: str) -> str:
    warm, cold = warm_split(trace_csv, kernel)
    if not warm:
        raise SystemExit(f"kernel {kernel} not found in {trace_csv}")
    out = [f"`{kernel}` per dispatch: {len(warm)} warm, average {statistics.mean(warm):.2f} us, "
           f"median {statistics.median(warm):.2f} us"]
    if cold:
        out.append(f"; {len(cold)} after a cache flush, average {statistics.mean(cold):.2f} us")
    return "".join(out) + ".\n"


def _per_dispatch(rows, counter):
    d = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        key = (r["Dispatch_Id"], r["Kernel_Name"])
        d[key] = d.get(key, 0.0) + float(r["Counter_Value"])
    return d


def traffic_record(fetch_csv, write_csv, kernel, calib_mib, cmd_fetch, cmd_write):
    fetch = _per_dispatch(_counter_rows(fetch_csv), "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(write_csv), "WRITE_SIZE")
    calib_kib = calib_mib * 1024.0

    def calib(vals):
        # the copy is the copy-kernel dispatch whose reading is closest to calib_kib
        cands = [v for (did, name), v in vals.items() if "copyBuffer" in name or "copy" in name.lower()]
        if not cands:
            raise SystemExit("no copy-kernel dispatch found for calibration")
        return min(cands, key=lambda v: abs(v - calib_kib))

    f_cal, w_cal = calib(fetch), calib(write)
    f_fac, w_fac = calib_kib / f_cal, calib_kib / w_cal
    fk = [v for (did, name), v in fetch.items() if kernel in name]
    wk = [v for (did, name), v in write.items() if kernel in name]
    if not fk or not wk:
        raise SystemExit(f"kernel {kernel} not found in counter output")
    fetch_b = statistics.median(fk) * 1024.0 * f_fac
    write_b = statistics.median(wk) * 1024.0 * w_fac
    return {
        "kernel": kernel,
        "source_sha256": source_digest(kernel),
        "fetch_kib_per_launch_raw": statistics.median(fk),
        "write_kib_per_launch_raw": statistics.median(wk),
        "launches": [len(fk), len(wk)],
        "calibration": {"copy_mib": calib_mib, "fetch_kib_read": f_cal, "write_kib_read": w_cal,
                        "fetch_factor": f_fac, "write_factor": w_fac},
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "traffic_bytes_per_launch": fetch_b + write_b,
        "commands": {"fetch": cmd_fetch, "write": cmd_write},
    }


N_XCD = 8
N_SIMD = 1024


def mfma_markdown(path, kernel, alg_flops, cmd):
    rows = _counter_rows(path)
    per = {}
    for r in rows:
        if kernel not in r["Kernel_Name"]:
            continue
        d = per.setdefault(r["Dispatch_Id"], {"name": r["Kernel_Name"],
                                              "us": (int(r["End_Timestamp"]) -
                                                     int(r["Start_Timestamp"])) / 1e3})
        d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"kernel {kernel} not found in counter output")
    out = ["| dispatch | executed MFMA flops | / algorithmic | MFMA busy cycles | "
           "active cycles per XCD | MFMA utilisation | duration under the profiler (us) |",
           "|---|---|---|---|---|---|---|"]
    for did, d in sorted(per.items(), key=lambda kv: int(kv[0])):
        mops = sum(v for k, v in d.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS"))
        flops = mops * 512
        busy = d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0.0)
        active = d.get("GRBM_GUI_ACTIVE", 0.0) / N_XCD
        util = busy / (active * N_SIMD) if active else float("nan")
        out.append(f"| {did} | {flops:.4g} | {flops / alg_flops:.4f} | {busy:.4g} | {active:.4g} | "
                   f"{100 * util:.1f}% | {d['us']:.1f} |")
    name = next(iter(per.values()))["name"]
    return (f"Kernel: `{name}`\n\nCommand:\n\n```\n{cmd}\n```\n\n" + "\n".join(out) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--calib-mib", type=float, required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd-fetch", required=True)
    t.add_argument("--cmd-write", required=True)
    wsub = sub.add_parser("warm")
    wsub.add_argument("trace_csv")
    wsub.add_argument("--kernel", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("csv")
    m.add_argument("--kernel", required=True)
    m.add_argument("--algorithmic-flops", type=float, required=True)
    m.add_argument("--cmd", required=True)
    a = ap.parse_args(argv)
    if a.what == "stats":
        sys.stdout.write(stats_markdown(a.csv, a.cmd))
    elif a.what == "warm":
        sys.stdout.write(warm_markdown(a.trace_csv, a.kernel))
    elif a.what == "mfma":
        sys.stdout.write(mfma_markdown(a.csv, a.kernel, a.algorithmic_flops, a.cmd))
    else:
        rec = traffic_record(a.fetch, a.write, a.kernel, a.calib_mib, a.cmd_fetch, a.cmd_write)
        with open(a.out, "w") as f:
            json.dump(rec, f, indent=2)
            f.write("\n")
        print(json.dumps(rec, indent=2))


if __name__ == "__main__":
    main()
