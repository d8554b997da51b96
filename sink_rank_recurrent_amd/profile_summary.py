"""Summarise rocprofv3 CSV output into short text files.

    python -m sink_rank_recurrent_amd.profile_summary trace <kernel_stats.csv> <kernel_trace.csv> \
        --command "<the rocprofv3 command>" --out profiles/<name>.md
    python -m sink_rank_recurrent_amd.profile_summary counters --fetch <csv> --write <csv> \
        --copy-fetch <csv> --copy-write <csv> --bench-json <bench output> --source <kernel> \
        --commands "..." --out profiles/traffic_<kernel>_<workload>.json
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


def trace_summary(stats_csv: str, trace_csv: str, command: str, title: str,
                  window=None, window_group: str = "seed_step_kernel (lazy decay)"):
    rows = list(csv.DictReader(open(stats_csv)))
    top = 25
    lines = [f"# {title}", "", "Command:", "", "```", command, "```", "",
             f"The {min(top, len(rows))} kernels with the most total time, of {len(rows)}:", "",
             "| kernel | calls | avg us | total ms | share % |", "|---|---|---|---|---|"]
    for r in rows[:top]:
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
    if window is not None:
        # the dispatches [start, start + count) of one group, in launch order
        # (the benchmark's timed launches of its headline kernel)
        start, count = window
        rows = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]))
                      for r in csv.DictReader(open(trace_csv))
                      if re.search(GROUPS[window_group], r["Kernel_Name"]))
        sel = [e - b for b, e in rows[start:start + count]]
        if len(sel) != count:
            raise SystemExit(f"window {start}:{count} beyond the {len(rows)} dispatches")
        merged["window"] = {"group": window_group, "start": start, "count": count,
                            "avg_us": sum(sel) / count / 1e3}
        lines += ["", f"{window_group}, dispatches {start} .. {start + count - 1} in launch "
                  f"order (the timed launches): {count} dispatches, "
                  f"avg {sum(sel) / count / 1e3:.2f} us"]
    lines.append("")
    return "\n".join(lines), merged


def counter_totals(counter_csv: str, kernel_pat: str, window=None):
    """Per-dispatch sums of each counter over the dispatches of matching
    kernels; with window = (start, count) only those dispatches, in
    dispatch order."""
    per = defaultdict(lambda: defaultdict(float))
    for r in csv.DictReader(open(counter_csv)):
        if not re.search(kernel_pat, r["Kernel_Name"]):
            continue
        per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
    if window is not None:
        start, count = window
        keys = sorted(per)[start:start + count]
        if len(keys) != count:
            raise SystemExit(f"window {start}:{count} beyond the {len(per)} dispatches")
        per = {k: per[k] for k in keys}
    return per


def _window(text):
    if not text:
        return None
    a, b = text.split(":")
    return int(a), int(b)


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("stats")
    t.add_argument("trace")
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="rocprofv3 kernel trace")
    t.add_argument("--out", required=True)
    t.add_argument("--window", default=None,
                   help="START:COUNT -- also average one kernel group (--group) over these "
                        "dispatches in launch order")
    t.add_argument("--group", default="seed_step_kernel (lazy decay)", choices=sorted(GROUPS),
                   help="the kernel group --window counts")
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True, help="counter_collection.csv of the FETCH_SIZE run")
    c.add_argument("--write", required=True, help="counter_collection.csv of the WRITE_SIZE run")
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--copy-bytes", type=float, default=float(1 << 30))
    c.add_argument("--kernel", default=GROUPS["seed_step_kernel (lazy decay)"])
    c.add_argument("--source", required=True, help="kernel source whose hash is recorded")
    c.add_argument("--bench-json", required=True,
                   help="the JSON line bench.py printed in the profiled run: its algorithmic "
                        "bytes per launch, steps, warm-up steps and layers")
    c.add_argument("--window", default=None,
                   help="START:COUNT of the kernel's dispatches to average (default: the "
                        "bench line's timed launches, after its pre-roll and settle steps)")
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
        # only the dispatches of the stated size (a warm-up launch of one
        # unit is left out); the SQ counters may see part of the GPU, so the
        # per-wave figures divide by SQ_WAVES of the same dispatches
        grid = args.units * args.waves_per_unit * 64
        means = {}
        for path in args.csvs:
            rows = [r for r in csv.DictReader(open(path)) if re.search(args.kernel, r["Kernel_Name"])]
            if rows and "Grid_Size" in rows[0]:
                rows = [r for r in rows if int(float(r["Grid_Size"])) == grid]
            per = defaultdict(lambda: defaultdict(float))
            for r in rows:
                per[int(r["Dispatch_Id"])][r["Counter_Name"]] += float(r["Counter_Value"])
            names = sorted({k for d in per.values() for k in d})
            for name in names:
                vals = [d[name] for d in per.values() if name in d]
                means[name] = (sum(vals) / len(vals), len(vals))
        waves = means.get("SQ_WAVES", (None, 0))[0]
        lines = [f"# {args.title}", "", "Commands:", "", "```", args.command, "```", "",
                 f"Kernel: `{args.kernel}`, dispatches of {args.units} units "
                 f"({args.waves_per_unit} wave(s) per unit) only."]
        if waves:
            lines += ["", f"SQ_WAVES counts {waves:.0f} of the {args.units * args.waves_per_unit} "
                      f"waves of a dispatch ({waves / (args.units * args.waves_per_unit):.3f}): "
                      "the SQ counters see that share of the GPU, so the per-wave column "
                      "divides by SQ_WAVES."]
        lines += ["", "| counter | dispatches | mean per dispatch | per wave |", "|---|---|---|---|"]
        for name, (v, nd) in sorted(means.items()):
            pw = f"{v / waves:.4g}" if waves else "-"
            lines.append(f"| {name} | {nd} | {v:.4g} | {pw} |")
        lines.append("")
        with open(args.out, "w") as f:
            f.write("\n".join(lines))
        print("\n".join(lines))
        return 0

    if args.cmd == "trace":
        text, merged = trace_summary(args.stats, args.trace, args.command, args.title,
                                     _window(args.window), args.group)
        with open(args.out, "w") as f:
            f.write(text)
        print(json.dumps(merged))
        return 0

    def mean_kib(path, pat, name, window=None):
        per = counter_totals(path, pat, window)
        vals = [d[name] for d in per.values() if name in d]
        return sum(vals) / len(vals), len(vals)

    line = None
    for text in open(args.bench_json).read().splitlines():
        if text.startswith("{"):
            line = json.loads(text)
    if line is None:
        raise SystemExit(f"no JSON line in {args.bench_json}")
    L = line["config"]["layers"]
    pre = line["breakdown"]["pre_roll_steps"]
    window = _window(args.window) or ((pre + line["warmup"]) * L, line["steps"] * L)
    fetch, nf = mean_kib(args.fetch, args.kernel, "FETCH_SIZE", window)
    write, nw = mean_kib(args.write, args.kernel, "WRITE_SIZE", window)
    algorithmic = line["roofline"]["algorithmic_bytes_per_launch"]
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
           "algorithmic_bytes_per_launch": algorithmic,
           "traffic_over_algorithmic": hbm / algorithmic,
           "dispatch_window": list(window),
           "bench_workload": line["config"]["workload"], "bench_layers": L,
           "bench_steps": line["steps"], "bench_warmup": line["warmup"],
           "kernel_source": os.path.relpath(args.source),
           "kernel_source_sha256_16": src_hash,
           "commands": args.commands}
    with open(args.out, "w") as f:
        json.dump(out, f, indent=1)
    print(json.dumps(out, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
