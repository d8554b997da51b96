"""Benchmark of the shallow-state decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]

A benchmark step is one decode token of the whole workload: for every
recurrent layer, one launch of the fused read-out + exact update kernel over
all of that layer's (request, head) units, and every W steps per layer the
compression of that layer's factors from R + W back to R columns.  The
default workload is the 36-layer stack: 36 recurrent layers x 32 heads x 256
resident requests of 128 x 128 Gated DeltaNet heads (R = 16, W = 32), all 36
layers' states resident in HBM at once (14.5 GB of factors at R + W), so no
layer's state is still in the memory-side cache when its next step comes.

Compression inside the timed region.  Each layer compresses every W steps
(SEED figures and tables, Fig. 1 (b) caption) on its own phase: layer l's
first window after the end-of-prefill conversion is W - floor(l W / L)
steps, every later one W.  So every timed step compresses about L / W
layers, and any K consecutive timed steps hold the compression work at its
true 1/W share per layer, whatever K is.  The compressions of a step run
after all its layer steps (each before that layer's next step).  An
untimed pre-roll of W steps (graphs replayed before the settle pass) takes
every layer past its shortened first window, so every settle and timed
compression is of the full R + W columns.

Timing.  The inputs of every timed step are drawn beforehand and resident
in HBM.  The bench steps are captured as HIP graphs from the same C-ABI
calls: one graph per run of step launches with no compression between them
(the L launches of one bench step on the staggered stack, W steps of a
single layer), one per run of compressions.  The W warm-up steps' graphs
are replayed first as an untimed settle pass (reported on its own,
`settle`), then the K timed steps' graphs, with a HIP event on the launch
stream before each graph and after the last, so no event sits between two
kernels of a graph.  `value` = head-steps (L x requests x heads x K) / the events' time
from the first timed graph to the end of the last.  The step kernel's
average launch duration is its graphs' event time / (L K); `roofline`
divides its algorithmic bytes per launch by that.

Also in the line: the dense-state baseline (dense_decode_step) on the same
stack, the lazily decayed and the 16-bit forms timed the same way, the
other four workloads (one layer each, timed over whole compression windows
after a settle window) in `workloads`, the end-of-prefill conversion, the
handoff of layer 0's converted states, their statistics, the library's
streaming-copy rate and the CPU oracle on a bounded sample (`cpu_baseline`).
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import copy
import hashlib
import json
import math
import os
import subprocess
import sys
import tempfile
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
MFMA_F32_PEAK_TFLOPS = 157.3  # MI355X dense fp32 matrix rate, vendor figure
# Merge delay of the per-request schedule variant: on the 36 resident layers
# D = 2 measured fastest of 1..12 (3.41 ms per bench step; 3.97 at D = 1,
# where every step launches a compression per layer, and 3.46-3.78 from 3
# to 12, where each step of delay holds one more column).
PER_REQUEST_DELAY = 2
DEFAULT_WORKLOAD = 5
STEP_SOURCE = os.path.join(ROOT, "sink_rank_recurrent_amd", "csrc", "seed_step.hip")
METRIC = ("decode head-steps/s + achieved HBM GB/s (% peak), sink+rank-R state update "
          "(whole job: every layer's step and its compression every W steps, phases staggered "
          "over the layers, all inside the timed region)")
# the machine's CPU share for one GPU: at most this many oracle processes
CPU_SHARE = 16


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes (what the method must move): a step reads a, r columns of
# U and V, the inputs and vbar; it writes a, all r + 1 columns of U (in-place
# decay plus the new column), one V column and o (fp32).
# ---------------------------------------------------------------------------

def step_bytes_per_unit(w, r: int, form: str = "in_place") -> float:
    """In place: U is read and written whole.  Lazy decay: U is only read,
    one new column is written, and the decay product (one float, or d_k for
    KDA) is read and written.  16-bit kept factors (lazy): the R kept
    columns are read at 2 bytes an entry, the r - R appended ones at 4."""
    s_in = 2 if w.in_dtype_name == "bf16" else 4
    g_bytes = 4 * w.d_k if w.rule == "kda" else 4
    beta_bytes = 0 if w.rule == "mamba2" else 4
    cols = 4 * (w.d_k + w.d_v) * r
    if form == "h16":
        cols = 2 * (w.d_k + w.d_v) * w.R + 4 * (w.d_k + w.d_v) * (r - w.R)
    read = 4 * w.d_k + cols + s_in * (2 * w.d_k + w.d_v) + g_bytes + beta_bytes
    read += 4 * w.d_v / w.batch          # vbar, shared by the requests of a head
    if form in ("lazy", "h16"):
        gam_bytes = 4 * w.d_k if w.rule == "kda" else 4
        read += gam_bytes
        write = 4 * w.d_k + 4 * w.d_k + 4 * w.d_v + 4 * w.d_v + gam_bytes
    else:
        write = 4 * w.d_k + 4 * w.d_k * (r + 1) + 4 * w.d_v + 4 * w.d_v
    return read + write


def dense_bytes_per_unit(w) -> float:
    s_in = 2 if w.in_dtype_name == "bf16" else 4
    g_bytes = 4 * w.d_k if w.rule == "kda" else 4
    beta_bytes = 0 if w.rule == "mamba2" else 4
    return 8 * w.d_k * w.d_v + s_in * (2 * w.d_k + w.d_v) + g_bytes + beta_bytes + 4 * w.d_v


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_file(w) -> str:
    return os.path.join(ROOT, "profiles", f"traffic_seed_step_{w.name}.json")


def load_traffic(w, steps: int, warmup: int):
    """HBM bytes per step-kernel launch from the committed counter summary
    of this very command (workload, timed and warm-up steps), or None if
    there is none or the step kernel's source changed since."""
    path = traffic_file(w)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(STEP_SOURCE):
        return None
    if t.get("bench_steps") != steps or t.get("bench_warmup") != warmup:
        return None
    return t.get("hbm_bytes_per_launch")


def counters_file(w) -> str:
    return os.path.join(ROOT, "profiles",
                        f"counters_compress_wave_{w.rule}_{w.batch}x{w.heads}_n{w.R + w.W}.md")


def load_compress_counters(w):
    """Per-unit instruction counts of the fp32 compression kernel from the
    committed rocprofv3 summary of this workload's compressions
    (profile_compress.sh), or None if there is none.  MFMA work does not
    depend on the data: it is fixed by n, R and the head shape."""
    import re
    path = counters_file(w)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"dispatches of (\d+) units \((\d+) wave", text)
    if not m:
        return None
    units, wpu = int(m.group(1)), int(m.group(2))
    rows = {}
    for name, per_dispatch, per_wave in re.findall(
            r"^\| (SQ_\w+) \| \d+ \| ([0-9.e+-]+) \| ([0-9.e+-]+) \|$", text, re.M):
        rows[name] = (float(per_dispatch), float(per_wave))
    if "SQ_INSTS_VALU_MFMA_MOPS_F32" not in rows or "SQ_INSTS_VALU" not in rows:
        return None
    return {"file": os.path.relpath(path, ROOT),
            # one MOP of this counter is 512 fp32 flops
            "mfma_flops_per_unit": rows["SQ_INSTS_VALU_MFMA_MOPS_F32"][0] * 512 / units,
            "valu_insts_per_unit": rows["SQ_INSTS_VALU"][1] * wpu,
            "mfma_insts_per_unit": rows["SQ_INSTS_MFMA"][1] * wpu if "SQ_INSTS_MFMA" in rows
            else None}


def compression_roofline(w, units: int, avg_us):
    """The compression kernel against both of its ceilings: HBM (it reads
    n = R + W columns of U and V and writes R) and fp32 MFMA (its dense
    products, counted by rocprofv3).  It is bound by neither: its serial
    Cholesky, Householder and eigen-solver chains bound it."""
    if not avg_us:
        return None
    n = w.R + w.W
    bytes_unit = 4 * (w.d_k + w.d_v) * (n + w.R)
    s = avg_us * 1e-6
    rec = {"kernel": "compress_wave_kernel", "columns": n, "units_per_launch": units,
           "avg_launch_us": avg_us, "bytes_per_unit": bytes_unit,
           "achieved_GBs": bytes_unit * units / s / 1e9,
           "hbm_frac": bytes_unit * units / s / 1e9 / HBM_PEAK_GBS}
    c = load_compress_counters(w)
    if c:
        tf = c["mfma_flops_per_unit"] * units / s / 1e12
        rec.update({"mfma_flops_per_unit": c["mfma_flops_per_unit"],
                    "mfma_achieved_TFLOPs": tf, "mfma_peak_TFLOPs": MFMA_F32_PEAK_TFLOPS,
                    "mfma_frac": tf / MFMA_F32_PEAK_TFLOPS,
                    "valu_insts_per_unit": c["valu_insts_per_unit"],
                    "mfma_insts_per_unit": c["mfma_insts_per_unit"], "counters": c["file"]})
    return rec


# ---------------------------------------------------------------------------
# the layer stack
# ---------------------------------------------------------------------------

class Spec:
    """Host-side description of a workload (no torch types), for the byte
    account and the CPU worker."""

    def __init__(self, w):
        self.name, self.rule, self.batch, self.heads = w.name, w.rule, w.batch, w.heads
        self.layers, self.d_k, self.d_v, self.R, self.W = w.layers, w.d_k, w.d_v, w.R, w.W
        self.in_dtype_name = "bf16" if "bfloat16" in str(w.in_dtype) else "f32"
        self.units = w.batch * w.heads


def layer_phases(L: int, W: int) -> list:
    """Compression phase of each layer: layer l's first window after the
    conversion is W - phase[l] steps, so the L layers' compressions spread
    evenly over the W steps of a window."""
    return [(l * W) // L for l in range(L)]


def prefill_layers(w, layers: int, dev: str):
    """vbar and the dense state after the 512-step dense prefill, per layer."""
    import torch
    from sink_rank_recurrent_amd import binding
    from sink_rank_recurrent_amd import workloads as wl

    vbars, Ss = [], []
    o = torch.empty(w.batch, w.heads, w.d_v, device=dev)
    for layer in range(layers):
        vbar = wl.make_vbar(w.heads, w.d_v, w.seed, layer, dev)
        S = torch.zeros(w.batch, w.heads, w.d_k, w.d_v, device=dev)
        for t in range(-w.prefill, 0):
            x = wl.workload_step(w, vbar, t, layer, dev)
            binding.dense_decode_step(w.rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        vbars.append(vbar)
        Ss.append(S)
    return vbars, Ss


def make_inputs(w, vbars, n_steps: int, dev: str):
    """inputs[l][t]: the resident inputs of decode step t of layer l."""
    from sink_rank_recurrent_amd import workloads as wl

    return [[wl.workload_step(w, vbars[l], t, l, dev) for t in range(n_steps)]
            for l in range(len(vbars))]


def make_states(w, form: str, vbars, Ss, phases, dev: str, timed_conversion: bool = False):
    """One state per layer, converted from its dense state (first window
    W - phase).  Returns (states, conversion ms or None)."""
    import torch
    from sink_rank_recurrent_amd import binding

    states = []
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    conv_ms = 0.0
    for l, (vbar, S) in enumerate(zip(vbars, Ss)):
        fw = w.W - phases[l]
        if form == "h16":
            st = binding.ShallowState16(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W, vbar,
                                        store=torch.float16, rounding="nearest", device=dev,
                                        first_window=fw)
        else:
            st = binding.ShallowState(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W, vbar,
                                      device=dev, lazy=(form == "lazy"), first_window=fw)
        if timed_conversion:
            ev[0].record()
            st.from_dense(S)
            ev[1].record()
            torch.cuda.synchronize()
            conv_ms += ev[0].elapsed_time(ev[1])
        else:
            st.from_dense(S)
        states.append(st)
    return states, (conv_ms if timed_conversion else None)


def plan(states, n: int):
    """The next n bench steps: for each, the (layer, r) of its step launches
    and the (layer, r) of the compressions that follow them.  Returns
    (plan, final r per layer, final limit per layer); the states are not
    touched."""
    r = [st.r for st in states]
    lim = [st.limit for st in states]
    out = []
    for _ in range(n):
        steps = [(l, r[l]) for l in range(len(states))]
        comps = []
        for l in range(len(states)):
            r[l] += 1
            if r[l] >= lim[l]:
                comps.append((l, r[l]))
                r[l] = states[l].R
                lim[l] = states[l].cap
        out.append((steps, comps))
    return out, r, lim


def warm_compress_instances(w, form: str, rs, dev: str) -> None:
    """Run every compression instance the plan uses once, eagerly, on a
    one-unit scratch state, so that its one-time LDS attribute is set before
    any graph capture."""
    import torch
    from sink_rank_recurrent_amd import binding

    vbar = torch.ones(w.heads, w.d_v, device=dev)
    for r in sorted(set(rs)):
        if form == "h16":
            st = binding.ShallowState16(w.rule, 1, w.heads, w.d_k, w.d_v, w.R, w.W, vbar,
                                        device=dev)
        else:
            st = binding.ShallowState(w.rule, 1, w.heads, w.d_k, w.d_v, w.R, w.W, vbar,
                                      device=dev, lazy=(form == "lazy"))
        st.launch_compress(r)
    torch.cuda.synchronize()


def _ops(pl, lo: int, hi: int, overlap: bool, pending):
    """The bench steps lo .. hi-1 of a plan as a list of operations:
    ("steps", [(t, l, r), ...]) for every maximal run of step launches that
    nothing has to come between, and then
      * overlap: ("fork", l, r) right after layer l's step launch whose
        window ends there (its compression, on the side stream), and
        ("wait", l) right before layer l's next step launch (the launch
        stream waits for that compression);
      * otherwise: ("compress", [(l, r), ...]) after the L step launches of
        the bench step, on the launch stream.
    `pending` (a set of layers whose compression is in flight) is updated."""
    ops, cur = [], []

    def flush():
        if cur:
            ops.append(("steps", list(cur)))
            cur.clear()

    for t in range(lo, hi):
        steps, comps = pl[t]
        comp_of = dict(comps)
        for l, r in steps:
            if overlap and l in pending:
                flush()
                ops.append(("wait", l))
                pending.discard(l)
            cur.append((t, l, r))
            if overlap and l in comp_of:
                flush()
                ops.append(("fork", l, comp_of[l]))
                pending.add(l)
        if not overlap and comps:
            flush()
            ops.append(("compress", comps))
    flush()
    return ops


def run_stack(w, states, inputs, outs, n_pre: int, n_settle: int, n_timed: int, form: str,
              dev: str, joins=None, join_bufs=None, overlap: bool = True):
    """Run n_pre + n_settle + n_timed bench steps of the layer stack: each
    run of step launches is one HIP graph, replayed on the launch stream.
    With overlap, a layer's compression runs on a side stream (default
    priority), forked right after the step launch that ends its window and
    joined right before that layer's next step launch, so it overlaps the
    other layers' steps; without, the compressions of a bench step follow
    its L step launches on the launch stream.  The pre-roll and the settle
    steps run first; in the timed steps an event pair on the launch stream
    brackets every graph (the step launches' time), one on the side stream
    every compression, and the timed region starts with no compression in
    flight and ends when the last compression it started has finished.  joins: {bench step: int32 slots} -- before its
    step launch at that bench step, each layer takes the requests of
    join_bufs[layer] into those slots (seed_join_states, at the column count
    the plan gives it)."""
    import torch
    from sink_rank_recurrent_amd import binding

    pl, r_end, lim_end = plan(states, n_pre + n_settle + n_timed)
    warm_compress_instances(w, form, [r for _, comps in pl for _, r in comps], dev)
    fns = [st.bind_step(outs[l]) for l, st in enumerate(states)]
    main = torch.cuda.current_stream()
    side = torch.cuda.Stream()
    pending = set()
    phases = [_ops(pl, 0, n_pre, overlap, pending),
              _ops(pl, n_pre, n_pre + n_settle, overlap, pending)]
    pending.clear()   # joined before the timed region (below)
    phases.append(_ops(pl, n_pre + n_settle, n_pre + n_settle + n_timed, overlap, pending))

    def capture(items):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t, l, r in items:
                if joins is not None and t in joins:
                    st = states[l]
                    binding.seed_join_states(st.rule, join_bufs[l], st.a, st.U, st.V, st.gam,
                                             st.R, r, joins[t])
                x = inputs[l][t]
                fns[l](x["q"], x["k"], x["v"], x["g"], x["beta"], r)
        return g

    graphs = [[capture(op[1]) if op[0] == "steps" else None for op in ops] for ops in phases]
    torch.cuda.synchronize()

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    done = {}
    rec = {"step": [], "comp": [], "all_comp": []}

    def execute(ops, gs, timed):
        for op, g in zip(ops, gs):
            if op[0] == "steps":
                if timed:
                    a, b = ev(), ev()
                    a.record(main)
                    g.replay()
                    b.record(main)
                    rec["step"].append((a, b, [r for _, _, r in op[1]]))
                else:
                    g.replay()
            elif op[0] == "wait":
                main.wait_event(done.pop(op[1]))
            elif op[0] == "fork":
                l, r = op[1], op[2]
                f = torch.cuda.Event()
                f.record(main)
                side.wait_event(f)
                a, b = ev(), ev()
                a.record(side)
                states[l].launch_compress(r, stream=side)
                b.record(side)
                done[l] = b
                rec["all_comp"].append((a, b))
                if timed:
                    rec["comp"].append((a, b, r))
            else:
                for l, r in op[1]:
                    a, b = ev(), ev()
                    a.record(main)
                    states[l].launch_compress(r)
                    b.record(main)
                    if timed:
                        rec["comp"].append((a, b, r))

    execute(phases[0], graphs[0], False)
    s0, s1 = ev(), ev()
    s0.record(main)
    execute(phases[1], graphs[1], False)
    # the timed region starts with no compression in flight (and ends after
    # the last one it started): none of the settle pass's work is counted
    for l in list(done):
        main.wait_event(done.pop(l))
    s1.record(main)
    t0, t1 = ev(), ev()
    t0.record(main)
    n_fork0 = len(rec["comp"])
    execute(phases[2], graphs[2], True)
    # the region ends when the compressions it started have finished
    for l in list(done):
        main.wait_event(done.pop(l))
    t1.record(main)
    torch.cuda.synchronize()
    for l, st in enumerate(states):
        st.r, st.limit = r_end[l], lim_end[l]
    step_ms = sum(a.elapsed_time(b) for a, b, _ in rec["step"])
    comp_ms = sum(a.elapsed_time(b) for a, b, _ in rec["comp"])
    timed_pl = pl[n_pre + n_settle:]
    step_r = [r for steps, _ in timed_pl for _, r in steps]
    comp_r = [r for _, _, r in rec["comp"]]
    assert n_fork0 == 0 and step_r == [r for _, _, rs in rec["step"] for r in rs]
    # the graphs of step launches during which no compression ran (events of
    # both streams on the one device clock, from the timed region's start)
    comp_iv = [(t0.elapsed_time(a), t0.elapsed_time(b)) for a, b in rec["all_comp"]]
    clear_ms, clear_r = 0.0, []
    for a, b, rs in rec["step"]:
        sa, sb = t0.elapsed_time(a), t0.elapsed_time(b)
        if all(cb <= sa or ca >= sb for ca, cb in comp_iv):
            clear_ms += sb - sa
            clear_r += rs
    return {"elapsed_ms": t0.elapsed_time(t1), "step_ms": step_ms, "compress_ms": comp_ms,
            "compressions": len(comp_r), "step_r": step_r, "compress_r": comp_r,
            "settle_ms": s0.elapsed_time(s1), "settle_steps": n_settle, "timed_steps": n_timed,
            "graphs": sum(1 for op in phases[2] if op[0] == "steps"),
            "pre_roll_steps": n_pre, "compress_columns": sorted(set(comp_r)),
            "overlap": overlap, "clear_step_ms": clear_ms, "clear_step_r": clear_r}


def summarise(spec, res, form: str, L: int) -> dict:
    """Whole-job rate, step-kernel roofline and compression share of one
    run_stack result."""
    units = spec.units
    n_launch = len(res["step_r"])
    step_bytes = sum(step_bytes_per_unit(spec, r, form) for r in res["step_r"]) * units
    avg_launch_s = res["step_ms"] / 1e3 / n_launch
    achieved = step_bytes / n_launch / avg_launch_s / 1e9
    el = res["elapsed_ms"] / 1e3
    n_comp = res["compressions"]
    return {
        "value": L * units * res["timed_steps"] / el,
        "ms_per_step": res["elapsed_ms"] / res["timed_steps"],
        "step_kernel_avg_us": avg_launch_s * 1e6,
        "step_launches": n_launch,
        "step_bytes_per_head_step": step_bytes / n_launch / units,
        "step_algorithmic_bytes_per_launch": step_bytes / n_launch,
        "step_achieved_GBs": achieved,
        "step_frac_of_peak": achieved / HBM_PEAK_GBS,
        "step_only_head_steps_per_s": units * n_launch / (res["step_ms"] / 1e3),
        # the same over the graphs of step launches with no compression
        # running beside them
        "step_clear_launches": len(res["clear_step_r"]),
        "step_clear_avg_us": (res["clear_step_ms"] * 1e3 / len(res["clear_step_r"])
                              if res["clear_step_r"] else None),
        "step_clear_achieved_GBs": (sum(step_bytes_per_unit(spec, r, form)
                                        for r in res["clear_step_r"]) * units
                                    / (res["clear_step_ms"] / 1e3) / 1e9
                                    if res["clear_step_r"] else None),
        "compressions": n_comp,
        "compress_avg_us": res["compress_ms"] * 1e3 / n_comp if n_comp else None,
        # on the launch stream the compressions' time is a share of the
        # elapsed time; overlapped on the side stream it is not
        "compress_share_of_time": (None if res["overlap"]
                                   else res["compress_ms"] / res["elapsed_ms"]),
        "compressions_overlapped": res["overlap"],
        "compressions_per_layer_step": n_comp / (L * res["timed_steps"]),
        "graphs_replayed": res["graphs"],
        "pre_roll_steps": res["pre_roll_steps"],
        "compress_columns": res["compress_columns"],
        "settle": {"steps": res["settle_steps"],
                   "ms_per_step": (res["settle_ms"] / res["settle_steps"]
                                   if res["settle_steps"] else None)},
    }


def run_dense(w, Ss, inputs, outs, t0: int, n_settle: int, n_timed: int) -> dict:
    """The dense-state baseline over the same layers and inputs: the settle
    steps and the timed steps captured as one HIP graph each (the L dense
    launches of every step, in order), the settle graph replayed first."""
    import torch
    from sink_rank_recurrent_amd import binding

    def capture(ts):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for t in ts:
                for l, S in enumerate(Ss):
                    x = inputs[l][t]
                    binding.dense_decode_step(w.rule, S, x["q"], x["k"], x["v"], x["g"],
                                              x["beta"], outs[l])
        return g

    g_settle = capture(range(t0, t0 + n_settle)) if n_settle else None
    g_timed = capture(range(t0 + n_settle, t0 + n_settle + n_timed))
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    e[0].record()
    if g_settle is not None:
        g_settle.replay()
    e[1].record()
    g_timed.replay()
    e[2].record()
    torch.cuda.synchronize()
    return {"elapsed_ms": e[1].elapsed_time(e[2]), "settle_ms": e[0].elapsed_time(e[1])}


def dense_summary(spec, d, L: int, n_timed: int) -> dict:
    units = spec.units
    el = d["elapsed_ms"] / 1e3
    avg = el / (L * n_timed)
    return {"value": L * units * n_timed / el, "unit": "head-steps/s",
            "ms_per_step": d["elapsed_ms"] / n_timed,
            "bytes_per_head_step": dense_bytes_per_unit(spec), "kernel_avg_us": avg * 1e6,
            "achieved_GBs": dense_bytes_per_unit(spec) * units / avg / 1e9,
            "frac_of_peak": dense_bytes_per_unit(spec) * units / avg / 1e9 / HBM_PEAK_GBS}


# ---------------------------------------------------------------------------
# the CPU baseline: the oracle in separate processes
# ---------------------------------------------------------------------------

def cpu_worker_main(path: str) -> int:
    """One oracle process (one thread): the factored mode (Lemma 2 steps,
    compression every W) on its units until its budget is spent, then the
    dense mode (the dense recurrence) on the same units.  Prints one JSON
    line of counts and times.  Never touches the GPU."""
    import numpy as np

    import oracle

    z = np.load(path)
    rule = str(z["rule"])
    R, W = int(z["R"]), int(z["W"])
    bf, bd = float(z["budget_factored"]), float(z["budget_dense"])
    a, U, V, vb, S = z["a"], z["U"], z["V"], z["vb"], z["S"]
    xs = [{k: (None if k == "beta" and z["beta"].size == 0 else z[k][i])
           for k in ("q", "k", "v", "g", "beta")} for i in range(z["q"].shape[0])]
    done = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < bf:
        x = xs[done % len(xs)]
        a, U, V, _ = oracle.seed_step(rule, a, U, V, vb, x["q"], x["k"], x["v"], x["g"],
                                      x["beta"])
        if U.shape[-1] >= R + W:
            U, V = oracle.compress(U, V, R)
        done += 1
    el_f = time.perf_counter() - t0
    dd = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < bd:
        x = xs[dd % len(xs)]
        S, _ = oracle.dense_step(rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"])
        dd += 1
    el_d = time.perf_counter() - t0
    print(json.dumps({"units": int(a.shape[0]), "factored_steps": done, "factored_s": el_f,
                      "dense_steps": dd, "dense_s": el_d}), flush=True)
    return 0


def cpu_baseline(spec, snap, budget_f: float, budget_d: float, workers: int) -> dict:
    """The oracle as it stands on a bounded sample of the workload: `workers`
    child processes (plain subprocesses, one thread each, none touching the
    GPU), each with its own slice of the sampled units, all at once; every
    child is waited for, so none outlives the benchmark."""
    import numpy as np

    a, U, V, vb, S, xs = snap
    n = a.shape[0]
    per = n // workers
    tmp = tempfile.mkdtemp(prefix="seed_cpu_")
    env = dict(os.environ, OMP_NUM_THREADS="1", OPENBLAS_NUM_THREADS="1", MKL_NUM_THREADS="1",
               HIP_VISIBLE_DEVICES="", ROCR_VISIBLE_DEVICES="", CUDA_VISIBLE_DEVICES="")
    procs = []
    try:
        for p in range(workers):
            sl = slice(p * per, (p + 1) * per)
            path = os.path.join(tmp, f"w{p}.npz")
            stack = lambda key: np.stack([x[key][sl] for x in xs])  # noqa: E731
            np.savez(path, rule=spec.rule, R=spec.R, W=spec.W, budget_factored=budget_f,
                     budget_dense=budget_d, a=a[sl], U=U[sl], V=V[sl], vb=vb[sl], S=S[sl],
                     q=stack("q"), k=stack("k"), v=stack("v"), g=stack("g"),
                     beta=(np.zeros(0) if xs[0]["beta"] is None else stack("beta")))
            procs.append(subprocess.Popen([sys.executable, os.path.abspath(__file__),
                                           "--cpu-worker", path], stdout=subprocess.PIPE,
                                          env=env, cwd=ROOT, text=True))
        res = []
        for pr in procs:
            out, _ = pr.communicate()
            if pr.returncode != 0:
                raise RuntimeError(f"CPU oracle worker failed with status {pr.returncode}")
            res.append(json.loads(out.strip().splitlines()[-1]))
    finally:
        for pr in procs:
            if pr.poll() is None:
                pr.kill()
                pr.wait()
        for f in os.listdir(tmp):
            os.remove(os.path.join(tmp, f))
        os.rmdir(tmp)
    f_rates = [r["units"] * r["factored_steps"] / r["factored_s"] for r in res]
    d_rates = [r["units"] * r["dense_steps"] / r["dense_s"] for r in res]
    steps = sum(r["factored_steps"] for r in res)
    return {"value": sum(f_rates), "unit": "head-steps/s", "cores": workers, "kind": "oracle",
            "single_thread_value": sum(f_rates) / workers,
            "dense_value": sum(d_rates), "dense_single_thread_value": sum(d_rates) / workers,
            "host_cpus_visible": os.cpu_count(),
            "host_cpus_usable": len(os.sched_getaffinity(0)),
            "host_cpu_share": CPU_SHARE,
            "sample": f"{workers} processes x {per} units of layer 0 of {spec.name} (one thread "
                      f"each, the box's CPU share for one GPU), {steps} factored decode steps in "
                      f"all (compression every {spec.W}) from the converted state for "
                      f"{budget_f:.0f} s, then the dense recurrence on the same units for "
                      f"{budget_d:.0f} s; fp64 numpy oracle; `single_thread_value` is the mean "
                      f"per-process (one-thread) rate"}


def cpu_snapshot(spec, state, S, vbar, xs_dev, n_units: int):
    """fp64 host copies of the first n_units units: converted state, dense
    state and step inputs (bf16 widened exactly)."""
    import torch

    f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
    units, cap = spec.units, state.cap
    a = f64(state.a.reshape(units, spec.d_k)[:n_units])
    U = f64(state.U.reshape(units, cap, spec.d_k)[:n_units, :state.r]).transpose(0, 2, 1)
    V = f64(state.V.reshape(units, cap, spec.d_v)[:n_units, :state.r]).transpose(0, 2, 1)
    vb = f64(vbar)[[u % spec.heads for u in range(n_units)]]
    Sn = f64(S.reshape(units, spec.d_k, spec.d_v)[:n_units])
    xs = [{k: (None if v is None else f64(v.reshape((units,) + v.shape[2:])[:n_units]))
           for k, v in x.items()} for x in xs_dev]
    return a, U, V, vb, Sn, xs


# ---------------------------------------------------------------------------

def achievable_copy_GBs(n_bytes: int = 1 << 31, reps: int = 5) -> float:
    """Read + write GB/s of the library's streaming copy (seed_stream_copy)
    over a buffer far larger than the 256 MB memory-side cache: what HBM
    delivers to a read-once, write-once kernel here, set beside the nominal
    8 TB/s."""
    import torch
    from sink_rank_recurrent_amd import binding

    src = torch.ones(n_bytes // 4, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    binding.stream_copy(src, dst)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        binding.stream_copy(src, dst)
    ev[1].record()
    torch.cuda.synchronize()
    gbs = 2 * n_bytes * reps / (ev[0].elapsed_time(ev[1]) / 1e3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbs


def copy_probe(n_bytes: int = 1 << 30, reps: int = 8) -> None:
    """A plain device copy of known size (calibration of the HBM byte
    counters): `reps` launches of dst.copy_(src) over n_bytes each."""
    import torch

    src = torch.ones(n_bytes // 4, device="cuda:0", dtype=torch.float32)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    print(json.dumps({"copy_probe_bytes_read_per_launch": n_bytes,
                      "copy_probe_bytes_written_per_launch": n_bytes, "launches": reps,
                      "GBs_read_plus_write": 2 * n_bytes * reps / el / 1e9}), flush=True)


def handoff_of(w, st, dev: str) -> dict:
    """Pack every request of one layer's converted states into one buffer,
    then unpack it into the same slots (20 times each, events around)."""
    import torch

    sel = torch.arange(w.batch, dtype=torch.int32, device=dev)
    buf = st.pack(sel)
    reps = 20
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    torch.cuda.synchronize()
    ev[0].record()
    for _ in range(reps):
        st.pack(sel, buf)
    ev[1].record()
    for _ in range(reps):
        st.unpack(buf, sel)
    ev[2].record()
    torch.cuda.synchronize()
    nbytes = buf.numel()
    t_pack = ev[0].elapsed_time(ev[1]) / reps / 1e3
    t_unpack = ev[1].elapsed_time(ev[2]) / reps / 1e3
    units = w.batch * w.heads
    return {"head_bytes": nbytes // units, "dense_head_bytes": 4 * w.d_k * w.d_v,
            "requests": w.batch, "buffer_bytes": nbytes,
            "pack_us": t_pack * 1e6, "unpack_us": t_unpack * 1e6,
            "pack_GBs": 2 * nbytes / t_pack / 1e9, "unpack_GBs": 2 * nbytes / t_unpack / 1e9}


def stats_of(w, S, vbar, dev: str) -> dict:
    """Statistics of one layer's prefilled dense states (the quantities the
    pages measure on model states), with the kernel's time."""
    import torch
    from sink_rank_recurrent_amd import binding

    nf = binding.lib().seed_stat_fields()
    rec = torch.empty(w.batch, w.heads, nf, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    binding.seed_state_stats(S, vbar, w.R, rec)
    e1.record()
    torch.cuda.synchronize()
    units = w.batch * w.heads
    r = rec.reshape(units, nf)[:, :len(binding.STAT_FIELDS)].double()
    med = {f: float(r[:, i].median()) for i, f in enumerate(binding.STAT_FIELDS)}
    return {"kernel_ms": e0.elapsed_time(e1), "units": units,
            "median_sink_share": med["sink_share"], "median_top_share": med["top_share"],
            "median_abs_cos_vstar_vbar": med["abs_cos_vstar_vbar"],
            "median_rank90": med["rank90"], "median_rank99": med["rank99"],
            "median_beyond_R_share": med["beyond_R_share"]}


def run_stagger_variants(w, spec, vbars, Ss, phases, inputs, outs, pre, settle, timed, dev,
                         aligned, overlap: bool = True, delays=None):
    """Requests that arrive at different times, on the stack, against the
    aligned lazily decayed form (`aligned`):
      * one global phase: an arriving request joins mid-window
        (seed_join_states) and compresses with the batch -- one request
        every 8 bench steps, joining every layer;
      * per-request schedules (seed_decode_step_sched): request b starts at
        phase b mod W and compresses on its own schedule, the snapshots of
        D consecutive steps compressed by one launch, D = PER_REQUEST_DELAY
        (or each of `delays`).
    The global phase runs its compressions as the aligned run does (on a
    side stream with overlap, else on the launch stream); the per-request
    schedules' smaller launches always run on a side stream."""
    import torch
    from sink_rank_recurrent_amd import binding

    out = []
    # one global phase with joins
    states, _ = make_states(w, "lazy", vbars, Ss, phases, dev)
    bufs = [st.pack(torch.zeros(1, dtype=torch.int32, device=dev)) for st in states]
    joins = {t: torch.tensor([(t // 8) % w.batch], dtype=torch.int32, device=dev)
             for t in range(pre, pre + settle + timed) if t % 8 == 0}
    res = run_stack(spec, states, inputs, outs, pre, settle, timed, "lazy", dev, joins, bufs,
                    overlap=overlap)
    r = summarise(spec, res, "lazy", len(states))
    n_join = sum(1 for t in joins if t >= pre + settle)
    out.append({"kind": "one global phase: arriving requests join mid-window "
                        "(seed_join_states) and compress with the batch",
                "value": r["value"], "unit": "head-steps/s", "ms_per_step": r["ms_per_step"],
                "joins_in_timed_steps": n_join, "requests_per_join": 1,
                "vs_aligned_lazy": r["value"] / aligned["value"] if aligned else None})
    log(f"{w.name} [global phase + joins]: {r['ms_per_step']:.3f} ms per step")
    del states, bufs
    torch.cuda.empty_cache()

    # per-request schedules
    cap_d = min(w.W - 1, 96 - w.R - w.W)
    for D in (delays or [PER_REQUEST_DELAY]):
        out.append(_per_request_run(w, spec, vbars, Ss, inputs, outs, pre, settle, timed, dev,
                                    aligned, min(D, cap_d)))
    return out


def _per_request_run(w, spec, vbars, Ss, inputs, outs, pre, settle, timed, dev, aligned, D):
    import torch
    from sink_rank_recurrent_amd import binding

    units = spec.units
    t_start = [-(b % w.W) - (w.W + D) for b in range(w.batch)]
    scheds = []
    for l, (vbar, S) in enumerate(zip(vbars, Ss)):
        # a launch holds the units of D phases only (512 of 8192 at D = 2),
        # so it leaves CUs to the steps: on a side stream it runs beside them
        # (at D = 4, 4.10 against 4.40 ms per step on the launch stream)
        st = binding.ScheduledState(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W, D, vbar,
                                    t_start, device=dev, side_streams=1)
        st.from_dense(S)
        scheds.append(st)
    for t in range(pre + settle):
        for l, st in enumerate(scheds):
            x = inputs[l][t]
            st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], outs[l])
    for st in scheds:
        st.join()
        st.pending.clear()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(pre + settle, pre + settle + timed):
            for l, st in enumerate(scheds):
                x = inputs[l][t]
                st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], outs[l])
        for st in scheds:
            st.join()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    el = e0.elapsed_time(e1) / 1e3
    value = len(scheds) * units * timed / el
    cols = [scheds[0].held_columns(b, t) for t in range(pre + settle, pre + settle + timed)
            for b in range(w.batch)]
    res = {"kind": "per-request schedules (seed_decode_step_sched): request b starts at "
                   "phase b mod W, the snapshots of D consecutive steps share one "
                   "compression launch", "D": D, "value": value, "unit": "head-steps/s",
           "ms_per_step": el * 1e3 / timed, "mean_columns": sum(cols) / len(cols),
           "vs_aligned_lazy": value / aligned["value"] if aligned else None}
    log(f"{w.name} [per-request schedules, D = {D}]: {el * 1e3 / timed:.3f} ms per step")
    del g, scheds
    torch.cuda.empty_cache()
    return res


def run_workload(w, layers: int, settle: int, timed: int, dev: str, forms, with_dense: bool,
                 keep_layer0: bool = False, no_stagger: bool = True, overlap: bool = False,
                 delays=None,
                 other_schedule: bool = False):
    """Prefill, convert and time `layers` layers of workload w in every form
    of `forms` (compressions overlapped on a side stream, or not), then the
    dense baseline; other_schedule adds the first form with the other
    choice (results["other_schedule"]).  Returns (results by form, dense,
    conversion ms, layer-0 objects for the CPU snapshot / handoff / stats)."""
    import torch

    spec = Spec(w)
    phases = layer_phases(layers, w.W)
    # an untimed pre-roll brings every layer past its first (shortened)
    # window, so that every settle and timed compression is of R + W columns
    pre = w.W if layers > 1 else 0
    vbars, Ss = prefill_layers(w, layers, dev)
    log(f"{w.name}: prefilled {layers} layer(s) x {spec.units} units")
    inputs = make_inputs(w, vbars, pre + settle + timed, dev)
    outs = [torch.empty(w.batch, w.heads, w.d_v, device=dev) for _ in range(layers)]
    results, conv_ms, layer0 = {}, None, None
    for form in forms:
        states, cm = make_states(w, form, vbars, Ss, phases, dev,
                                 timed_conversion=(form == forms[0]))
        if cm is not None:
            conv_ms = cm
        if keep_layer0 and form == forms[0]:
            # layer 0's converted and dense states as they are before any
            # timed step (copies: the runs below move the originals on)
            st0 = copy.copy(states[0])
            st0.a, st0.U, st0.V = states[0].a.clone(), states[0].U.clone(), states[0].V.clone()
            layer0 = {"state": st0, "S": Ss[0].clone(), "vbar": vbars[0],
                      "inputs": inputs[0][:min(pre + settle + timed, 64)]}
        res = run_stack(spec, states, inputs, outs, pre, settle, timed, form, dev,
                        overlap=overlap)
        results[form] = summarise(spec, res, form, layers)
        log(f"{w.name} [{form}]: {results[form]['ms_per_step']:.3f} ms per step, "
            f"{results[form]['compressions']} compressions in {timed} timed steps")
        del states
        torch.cuda.empty_cache()
    if other_schedule and layers > 1:
        form = forms[0]
        states, _ = make_states(w, form, vbars, Ss, phases, dev)
        res = run_stack(spec, states, inputs, outs, pre, settle, timed, form, dev,
                        overlap=not overlap)
        results["other_schedule"] = summarise(spec, res, form, layers)
        log(f"{w.name} [{form}, compressions "
            f"{'on the launch stream' if overlap else 'on a side stream'}]: "
            f"{results['other_schedule']['ms_per_step']:.3f} ms per step")
        del states
        torch.cuda.empty_cache()
    if "lazy" in forms and layers > 1 and not no_stagger:
        results["stagger"] = run_stagger_variants(w, spec, vbars, Ss, phases, inputs, outs, pre,
                                                  settle, timed, dev, results.get("lazy"),
                                                  overlap=overlap, delays=delays)
    dense = None
    if with_dense:
        d = run_dense(w, Ss, inputs, outs, pre, settle, timed)
        dense = dense_summary(spec, d, layers, timed)
        log(f"{w.name} [dense]: {dense['ms_per_step']:.3f} ms per step")
    return results, dense, conv_ms, layer0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--layers", type=int, default=None,
                    help="recurrent layers resident and stepped per token (default: the "
                         "workload's own count)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of the oracle's factored mode per process")
    ap.add_argument("--cpu-dense-budget", type=float, default=5.0,
                    help="seconds of the oracle's dense mode per process")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="oracle processes (default: the usable cores, at most 16)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-variant", action="store_true",
                    help="skip the lazily decayed and 16-bit forms")
    ap.add_argument("--no-sub", action="store_true",
                    help="skip the other workloads' entries")
    ap.add_argument("--stagger-d", type=lambda x: [int(v) for v in x.split(",")], default=None,
                    help="merge delays D of the per-request schedule variant (comma list; "
                         "default: PER_REQUEST_DELAY)")
    ap.add_argument("--overlap", action="store_true",
                    help="run each layer's compression on a side stream, beside the other "
                         "layers' steps (default: on the launch stream after its bench step; "
                         "the overlapped run of the same form is reported as a variant)")
    ap.add_argument("--cpu-worker", default=None, help=argparse.SUPPRESS)
    args = ap.parse_args()

    if args.cpu_worker:
        return cpu_worker_main(args.cpu_worker)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the shallow-state path has no cross-GPU exchange and "
              "this build runs on a single MI355X; --gpus must be 1", file=sys.stderr)
        return 2
    if args.steps < 1 or args.warmup < 0:
        print("need --steps >= 1 and --warmup >= 0", file=sys.stderr)
        return 2

    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    from sink_rank_recurrent_amd import binding
    from sink_rank_recurrent_amd import workloads as wl

    if args.copy_probe:
        copy_probe()
        return 0

    dev = "cuda:0"
    torch.cuda.set_device(0)
    binding.lib()
    w = wl.WORKLOADS[args.workload]
    L = args.layers if args.layers is not None else w.layers
    spec = Spec(w)
    steps, warmup = args.steps, args.warmup
    log(f"workload {w.name}: {L} layer(s) x {spec.units} units, {steps} timed steps after "
        f"{warmup} settle steps")
    # the reported form first: U decayed lazily (fp32 factors); the in-place
    # decay and the 16-bit kept factors are variants
    forms = ["lazy"] if args.no_variant else ["lazy", "in_place", "h16"]
    overlap = args.overlap
    results, dense, conv_ms, layer0 = run_workload(w, L, warmup, steps, dev, forms,
                                                   not args.no_dense, keep_layer0=True,
                                                   no_stagger=args.no_variant, overlap=overlap,
                                                   other_schedule=not args.no_variant,
                                                   delays=args.stagger_d)
    head = results[forms[0]]

    handoff = stats = None
    if not args.no_variant:
        handoff = handoff_of(w, layer0["state"], dev)
        stats = stats_of(w, layer0["S"], layer0["vbar"], dev)
        log(f"handoff: pack {handoff['pack_us']:.1f} us, unpack {handoff['unpack_us']:.1f} us; "
            f"statistics {stats['kernel_ms']:.1f} ms")

    workers = 0
    snap = None
    if not args.no_cpu:
        workers = args.cpu_workers or min(CPU_SHARE, len(os.sched_getaffinity(0)))
        workers = max(1, min(workers, spec.units // 16))
        n_cpu = min(spec.units, 64 * workers) // workers * workers
        snap = cpu_snapshot(spec, layer0["state"], layer0["S"], layer0["vbar"],
                            layer0["inputs"], n_cpu)
    del layer0
    torch.cuda.empty_cache()

    subs = {}
    if not args.no_sub:
        for num in (1, 2, 3, 4):
            if num == args.workload:
                continue
            ws = wl.WORKLOADS[num]
            sp = Spec(ws)
            n_timed = ws.W * max(1, math.ceil(steps / ws.W))
            rs, ds, cms, _ = run_workload(ws, 1, ws.W, n_timed, dev, forms, not args.no_dense,
                                          overlap=overlap)
            e = dict(rs[forms[0]])
            e["rule"] = "timed over whole windows: one settle window, then " \
                        f"{n_timed // ws.W} window(s) of {ws.W} steps and their compressions"
            e["us_per_step"] = e["ms_per_step"] * 1e3
            e["conversion_ms"] = cms
            e["dense_baseline"] = ds
            e["speedup_over_dense"] = e["value"] / ds["value"] if ds else None
            e["compression"] = compression_roofline(ws, sp.units, e["compress_avg_us"])
            for form, key in (("in_place", "in_place_decay_variant"),
                              ("h16", "fp16_factor_variant")):
                if form in rs and form != forms[0]:
                    e[key] = {"value": rs[form]["value"], "step_frac_of_peak":
                              rs[form]["step_frac_of_peak"],
                              "compress_avg_us": rs[form]["compress_avg_us"]}
            subs[ws.name] = e
            torch.cuda.empty_cache()

    cpu = None
    if snap is not None:
        cpu = cpu_baseline(spec, snap, args.cpu_budget, args.cpu_dense_budget, workers)
        log(f"cpu oracle: {cpu['value']:.1f} head-steps/s on {workers} processes")

    copy_gbs = achievable_copy_GBs()
    log(f"plain 2 GiB device copy: {copy_gbs:.0f} GB/s read + write")
    traffic = load_traffic(w, steps, warmup) if L == w.layers else None
    achieved = head["step_achieved_GBs"]

    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; no trace or checkpoint)",
        "config": {"workload": w.name, "rule": w.rule, "layers": L, "requests": w.batch,
                   "heads": w.heads, "heads_per_launch": spec.units,
                   "heads_total": L * spec.units, "d_k": w.d_k, "d_v": w.d_v, "R": w.R,
                   "W": w.W, "inputs": "bf16 q/k/v, fp32 gates" if spec.in_dtype_name == "bf16"
                   else "fp32", "prefill": w.prefill,
                   "decay_of_U": "lazy: U = Diag(gam) U~ with a running decay product per "
                                 "head, folded in below 2^-64 (fp32 factors)",
                   "schedule": "layer l compresses every W steps, first window W - floor(l W / L)",
                   "launch": ("one HIP graph per run of step launches; each layer's "
                              "compression on a side stream, forked after the step that ends "
                              "its window and joined before that layer's next step"
                              if overlap else
                              "one HIP graph per run of step launches, the compressions of a "
                              "bench step after its step launches on the same stream") +
                             "; pre-roll and settle pass first",
                   "resident_factor_bytes": L * spec.units * 4 * (w.d_k + w.d_v) * (w.R + w.W)
                   + L * spec.units * 4 * w.d_k},
        "roofline": {"bound": "hbm", "kernel": "seed_step_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": head["step_algorithmic_bytes_per_launch"],
                     "avg_launch_us": head["step_kernel_avg_us"],
                     "launches": head["step_launches"],
                     "without_concurrent_compression": {
                         "launches": head["step_clear_launches"],
                         "avg_launch_us": head["step_clear_avg_us"],
                         "achieved": head["step_clear_achieved_GBs"],
                         "frac": (head["step_clear_achieved_GBs"] / HBM_PEAK_GBS
                                  if head["step_clear_achieved_GBs"] else None)},
                     "achievable_copy_GBs": copy_gbs,
                     "frac_of_achievable": achieved / copy_gbs if copy_gbs else None},
        "cpu_baseline": cpu,
        "breakdown": {k: head[k] for k in ("step_kernel_avg_us", "step_bytes_per_head_step",
                                           "step_only_head_steps_per_s", "compressions",
                                           "compress_avg_us", "compress_share_of_time",
                                           "compressions_overlapped",
                                           "compressions_per_layer_step", "compress_columns",
                                           "pre_roll_steps")},
        "compression": compression_roofline(w, spec.units, head["compress_avg_us"]),
        "other_compression_schedule": (
            {k: results["other_schedule"][k]
             for k in ("value", "ms_per_step", "compressions_overlapped", "step_kernel_avg_us",
                       "step_clear_avg_us", "compress_avg_us", "compress_share_of_time")}
            if "other_schedule" in results else None),
        "settle": head["settle"],
        "dense_baseline": dense,
        "speedup_over_dense": head["value"] / dense["value"] if dense else None,
        "in_place_decay_variant": results.get("in_place"),
        "fp16_factor_variant": results.get("h16"),
        "staggered_schedule_variants": results.get("stagger"),
        "conversion": {"kernel": "compress_wave_kernel (conversion instance)", "ms": conv_ms,
                       "heads": L * spec.units,
                       "us_per_head": conv_ms * 1e3 / (L * spec.units) if conv_ms else None,
                       "what": "end-of-prefill sink split and rank-R truncation of every head "
                               "(once per request)"},
        "handoff": handoff,
        "state_stats": stats,
        "workloads": subs,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
