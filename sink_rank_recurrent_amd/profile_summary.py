"""Summarise rocprofv3 CSV output into short text files.

    python -m sink_rank_recurrent_amd.profile_summary trace <kernel_stats.csv> <kernel_trace.csv> \
        --command "<the rocprofv3 command>" --out profiles/<name>.md
    python -m sink_rank_recurrent_amd.profile_summary counters <counter_collection.csv> \
        --kernel seed_step_kernel --out <file.json> ...
    python -m sink_rank_recurrent_amd.profile_summary pmc <a.csv> [<b.csv> ...] \
        --kernel compress_wave_kernel --units 1024 --command "..." --out profiles/<name>.md

The step kernel is compiled once per column-slot count, so its dispatches
appear under several template names; `trace` also reports them merged.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

GROUPS = {
    "seed_step_kernel (U decayed in place)": r"seed_step_kernel<.*false, 0>",
    "seed_step_kernel (lazy decay)": r"seed_step_kernel<.*true, 0>",
    "seed_step_kernel (16-bit kept factors)": r"seed_step_kernel<.*true, [12]>",
    "compress_wave_kernel (fp32 factors)": r"compress_wave_kernel<.*, 0>",
    "compress_wave_kernel (16-bit kept factors)": r"compress_wave_kernel<.*, [12]>",
    "round_factors_kernel": r"round_factors_kernel<",
    "seed_step_kernel (per-request schedule)": r"seed_step_kernel<.*true, 3>",
    "compress_wave_kernel (per-request schedule)": r"compress_wave_kernel<.*, 3>",
    "handoff_kernel": r"handoff_kernel<",
    "stats_wave_kernel": r"stats_wave_kernel<",
    "compress_wave_kernel (end-of-prefill conversion)": r"compress_wave_kernel<.*, 4>",
    "dense_step_kernel": r"dense_step_kernel<",
}


def short(name: str) -> str:
    name = name.replace("void ", "").replace("(anonymous namespace)::", "")
    name = re.sub(r"\(.*$", "", name)
    return name[:110]


def trace_summary(stats_csv: str, trace_csv: str, command: str, title: str) -> str:
    rows = list(csv.DictReader(open(stats_csv)))
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             "| kernel | calls | avg us | total ms | share % |", "|---|---|---|---|---|"]
    for r in rows:
        lines.append(f"| `{short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                     f"{float(r['TotalDurationNs']) / 1e6:.3f} | {float(r['Percentage']):.2f} |")
    # merged groups from the per-dispatch trace
    dur = defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        for g, pat in GROUPS.items():
            if re.search(pat, r["Kernel_Name"]):
                dur[g].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    lines += ["", "Merged over template instances (from the per-dispatch trace):", "",
              "| kernel | dispatches | avg us | total ms |", "|---|---|---|---|"]
    merged = {}
    for g, d in dur.items():
        merged[g] = {"dispatches": len(d), "avg_us": sum(d) / len(d) / 1e3, "total_ms": sum(d) / 1e6}
        lines.append(f"| {g} | {len(d)} | {sum(d) / len(d) / 1e3:.2f} | {sum(d) / 1e6:.3f} |")
    lines.append("")
    return "\n".join(lines), merged


def counter_totals(counter_csv: str, kernel_pat: str):
    """Per-dispatch sums of each counter over the dispatches of matching kernels."""
    per = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(counter_csv)):
        if not re.search(kernel_pat, r["Kernel_Name"]):
            continue
        per[r["Dispatch_Id"]][r["Counter_Name"]] += float(r["Counter_Value"])
    return per


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("trace")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="rocprofv3 kernel trace")
    t.add_argument("--out", required=True)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True, help="counter_collection.csv of the FETCH_SIZE run")
    c.add_argument("--write", required=True, help="counter_collection.csv of the WRITE_SIZE run")
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    c.add_argument("--kernel", default=GROUPS["seed_step_kernel (U decayed in place)"])
    c.add_argument("--source", required=True, help="kernel source whose hash is recorded")
    c.add_argument("--algorithmic-bytes", type=float, required=True,
                   help="algorithmic bytes per launch of the profiled runs")
    c.add_argument("--commands", required=True)
    c.add_argument("--out", required=True)
    m = sub.add_parser("pmc")
    m.add_argument("csvs", nargs="+", help="counter_collection.csv files (one per pass)")
    m.add_argument("--kernel", required=True, help="regex of the kernel name")
    m.add_argument("--units", type=int, required=True, help="workgroups (units) per dispatch")
    m.add_argument("--waves-per-unit", type=int, default=1)
    m.add_argument("--command", required=True)
    m.add_argument("--title", default="rocprofv3 counters")
    m.add_argument("--out", required=True)
    args = ap.parse_args()

    if args.cmd == "pmc":
        means = {}
        for path in args.csvs:
            per = counter_totals(path, args.kernel)
            names = sorted({k for d in per.values() for k in d})
            for name in names:
                vals = [d[name] for d in per.values() if name in d]
                means[name] = (sum(vals) / len(vals), len(vals))
        lines = [f"# {args.title}", "", "Commands:", "", "```", args.command, "```", "",
                 f"Kernel: `{args.kernel}`, {args.units} units per dispatch.", "",
                 "| counter | dispatches | mean per dispatch | per unit |", "|---|---|---|---|"]
        for name, (v, nd) in sorted(means.items()):
            lines.append(f"| {name} | {nd} | {v:.4g} | {v / args.units:.4g} |")
        lines.append("")
        with open(args.out, "w") as f:
            f.write("\n".join(lines))
        print("\n".join(lines))
        return 0

    if args.cmd == "trace":
        text, merged = trace_summary(args.stats, args.trace, args.command, args.title)
        with open(args.out, "w") as f:
            f.write(text)
        print(json.dumps(merged))
        return 0

    def mean_kib(path, pat, name):
        per = counter_totals(path, pat)
        vals = [d[name] for d in per.values() if name in d]
        return sum(vals) / len(vals), len(vals)

    fetch, nf = mean_kib(args.fetch, args.kernel, "FETCH_SIZE")
    write, nw = mean_kib(args.write, args.kernel, "WRITE_SIZE")
    cf, _ = mean_kib(args.copy_fetch, r"copyBuffer", "FETCH_SIZE")
    cw, _ = mean_kib(args.copy_write, r"copyBuffer", "WRITE_SIZE")
    f_scale = args.copy_bytes / (cf * 1024.0)
    w_scale = args.copy_bytes / (cw * 1024.0)
    hbm = fetch * 1024.0 * f_scale + write * 1024.0 * w_scale
    src_hash = hashlib.sha256(open(args.source, "rb").read()).hexdigest()[:16]
    out = {"kernel": args.kernel, "dispatches": [nf, nw],
           "fetch_KiB_per_dispatch": fetch, "write_KiB_per_dispatch": write,
           "copy_probe_fetch_KiB": cf, "copy_probe_write_KiB": cw,
           "fetch_scale": f_scale, "write_scale": w_scale,
           "hbm_bytes_per_launch": hbm,
           "algorithmic_bytes_per_launch": args.algorithmic_bytes,
           "traffic_over_algorithmic": hbm / args.algorithmic_bytes,
           "kernel_source": os.path.relpath(args.source),
           "kernel_source_sha256_16": src_hash,
           "commands": args.commands}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
