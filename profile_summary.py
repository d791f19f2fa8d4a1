#!/usr/bin/env python3
"""Turn rocprofv3 CSV output of bench.py runs into the short summaries kept in profiles/.

  python profile_summary.py --workload c2 --path kv-centric \
      --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
      --copy-mib 1024 --commands CMDFILE

DIR arguments are rocprofv3 output directories written with --output-format csv:
  --trace       rocprofv3 --kernel-trace --stats     on bench.py --workload W --path P
  --fetch       rocprofv3 --pmc FETCH_SIZE           on the same bench.py command
  --write       rocprofv3 --pmc WRITE_SIZE           on the same bench.py command
  --copy-fetch  rocprofv3 --pmc FETCH_SIZE           on bench.py --copy-calibration MIB
  --copy-write  rocprofv3 --pmc WRITE_SIZE           on bench.py --copy-calibration MIB
  --util        rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil on the same bench.py command

Writes profiles/kernels_<workload>_<path>.md (per-kernel durations, dominant kernel
traffic, the exact commands) and profiles/traffic_<workload>_<path>.json (HBM bytes
per launch of the dominant kernel, FETCH_SIZE and WRITE_SIZE each scaled by what
the same counter reads for a plain device copy of known size; bench.py reports it
while the kernel sources still hash to the recorded digest).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)


def _csv(d: str, suffix: str):
    files = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def kernel_durations(trace_dir: str) -> dict:
    out = {}
    for r in _csv(trace_dir, "kernel_trace.csv"):
        dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3  # us
        out.setdefault(r["Kernel_Name"], []).append(dur)
    return out


def counter_per_dispatch(pmc_dir: str, counter: str, match: str) -> list:
    vals = []
    for r in _csv(pmc_dir, "counter_collection.csv"):
        if r["Counter_Name"] == counter and match in r["Kernel_Name"]:
            vals.append(float(r["Counter_Value"]))
    return vals


def short(name: str) -> str:
    name = name.replace("msa::(anonymous namespace)::", "").replace("void ", "")
    return name.split("(")[0]


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", required=True)
    ap.add_argument("--path", required=True)
    ap.add_argument("--trace", required=True)
    ap.add_argument("--fetch")
    ap.add_argument("--write")
    ap.add_argument("--copy-fetch")
    ap.add_argument("--copy-write")
    ap.add_argument("--copy-mib", type=int, default=1024)
    ap.add_argument("--commands", help="text file with the commands that produced the dirs")
    ap.add_argument("--out", default=os.path.join(ROOT, "profiles"))
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"])
    ap.add_argument("--util", help="rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil on the same command")
    args = ap.parse_args()

    import bench
    import workloads as wl

    durs = kernel_durations(args.trace)
    w = (wl.VARLEN_WORKLOADS[args.workload] if args.workload in wl.VARLEN_WORKLOADS
         else wl.WORKLOADS[args.workload])
    f8 = "true" if args.kv_dtype == "fp8" else "false"
    # q-centric names end with the wave count the launcher picked: matched as a prefix
    if w.paged:
        dom = {"paged-qcentric": f"qcentric_kernel<true, false, {f8},",
               "paged-decode": bench.decode_instance(w).replace("TEMP", "false"),
               "paged-dense-decode": bench.decode_instance(w, f8 == "true").replace("TEMP",
                                                                                    "false"),
               "paged-kv-centric": f"kvcentric_kernel<{w.qpk}, false, {f8}, true>",
               }[args.path]
    else:
        dom = {"q-centric": f"qcentric_kernel<false, false, {f8},",
               "kv-centric": f"kvcentric_kernel<{w.qpk}, false, {f8}, false>",
               "query-tile": f"tile_kernel<{w.qpk}, false>"}[args.path]
    tag = "" if args.kv_dtype == "bf16" else "-fp8"
    lines = [f"# Kernel profile: {w.name}, {args.path} path"
             + ("" if not tag else ", fp8 e4m3fn K/V cache"), ""]
    if args.commands:
        lines += ["Commands (run from the repository root on one MI355X):", "", "```"]
        lines += open(args.commands).read().strip().splitlines()
        lines += ["```", ""]
    lines += ["| kernel | calls | avg us | median us | min us | max us | total ms |",
              "|---|---|---|---|---|---|---|"]
    total = 0.0
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        if "elementwise" in name or "distribution" in name:
            continue
        total += sum(v)
        lines.append(f"| {short(name)} | {len(v)} | {statistics.mean(v):.1f} | "
                     f"{statistics.median(v):.1f} | {min(v):.1f} | {max(v):.1f} | "
                     f"{sum(v) / 1e3:.3f} |")
    dom_durs = [x for n, v in durs.items() if dom in n for x in v]
    dom_avg = statistics.mean(dom_durs) if dom_durs else None
    dom_med = statistics.median(dom_durs) if dom_durs else None
    full = [short(n) for n in durs if dom in n]
    if full:  # the instance as the trace names it
        dom_name = full[0]
    else:
        dom_name = dom
    lines += ["", f"Dominant kernel: `{dom_name}`, average {dom_avg:.1f} us per launch, median "
              f"{dom_med:.1f} us. Launch durations vary within one run: the first launches, and "
              "the first after each of bench.py's host-side phases, warm up, and the clock moves "
              "under sustained load; the median is the typical launch (under the profiler, a "
              "few per cent slower than without)." if dom_avg
              else f"Dominant kernel `{dom}` not found in the trace."]

    traffic = None
    if args.fetch and args.write and args.copy_fetch and args.copy_write:
        copy_bytes = args.copy_mib << 20
        cf = counter_per_dispatch(args.copy_fetch, "FETCH_SIZE", "copy")
        cw = counter_per_dispatch(args.copy_write, "WRITE_SIZE", "copy")
        kf = counter_per_dispatch(args.fetch, "FETCH_SIZE", dom)
        kw = counter_per_dispatch(args.write, "WRITE_SIZE", dom)
        if cf and cw and kf and kw:
            # bytes per counter unit: what the counter reads for a copy of known size
            fscale = copy_bytes / statistics.median(cf)
            wscale = copy_bytes / statistics.median(cw)
            fetch_b = statistics.median(kf) * fscale
            write_b = statistics.median(kw) * wscale
            traffic = fetch_b + write_b
            lines += ["", "HBM traffic of the dominant kernel per launch (rocprofv3 --pmc):", "",
                      f"- FETCH_SIZE {statistics.median(kf):.0f} (copy of {args.copy_mib} MiB reads "
                      f"{statistics.median(cf):.0f}; scale {fscale:.1f} B/unit) -> "
                      f"{fetch_b / 1e9:.3f} GB read",
                      f"- WRITE_SIZE {statistics.median(kw):.0f} (copy reads "
                      f"{statistics.median(cw):.0f}; scale {wscale:.1f} B/unit) -> "
                      f"{write_b / 1e9:.3f} GB written",
                      f"- total {traffic / 1e9:.3f} GB per launch"]
            # every kernel of the step: bytes per launch, and the rate over its traced time
            lines += ["", "HBM traffic of every kernel per launch (same scaling; rate = bytes / "
                      "average traced duration):", "",
                      "| kernel | read GB | written GB | TB/s |", "|---|---|---|---|"]
            for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
                f = counter_per_dispatch(args.fetch, "FETCH_SIZE", name)
                wr = counter_per_dispatch(args.write, "WRITE_SIZE", name)
                if not f or not wr:
                    continue
                rb = statistics.median(f) * fscale
                wb = statistics.median(wr) * wscale
                lines.append(f"| {short(name)} | {rb / 1e9:.3f} | {wb / 1e9:.3f} | "
                             f"{(rb + wb) / (statistics.mean(v) * 1e-6) / 1e12:.2f} |")
    if args.util:
        lines += ["", "Unit utilisation (rocprofv3 derived metrics, median over dispatches): "
                  "MfmaUtil = matrix-core busy cycles / (GPU-active cycles x SIMDs); VALUBusy and "
                  "LdsUtil = VALU- and LDS-active cycles / (GPU-active cycles x CUs).", "",
                  "| kernel | MfmaUtil % | VALUBusy % | LdsUtil % |", "|---|---|---|---|"]
        for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
            vals = [counter_per_dispatch(args.util, c, name) for c in
                    ("MfmaUtil", "VALUBusy", "LdsUtil")]
            if all(vals):
                lines.append(f"| {short(name)} | " + " | ".join(
                    f"{statistics.median(x):.1f}" for x in vals) + " |")
    os.makedirs(args.out, exist_ok=True)
    md = os.path.join(args.out, f"kernels_{args.workload}_{args.path}{tag}.md")
    with open(md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("wrote", md)
    if traffic is not None:
        js = os.path.join(args.out, f"traffic_{args.workload}_{args.path}{tag}.json")
        with open(js, "w") as fh:
            json.dump({"workload": w.name, "path": args.path, "kernel": dom_name,
                       "hbm_bytes_per_launch": traffic, "kernel_avg_us": dom_avg,
                       "kernel_median_us": dom_med,
                       "source_digest": bench.source_digest(dom)}, fh, indent=1)
            fh.write("\n")
        print("wrote", js)
    return 0


if __name__ == "__main__":
    sys.exit(main())
