"""Benchmark of the shallow-state decode path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload N]

One benchmark step is one decode step of every (request, head) unit of the
workload: the fused read-out + exact update kernel, plus the compression of
all units whenever R + W columns are held (every W steps), exactly as a
served decode loop would run them.  Inputs for every timed step are drawn
before timing and are resident in HBM; the state starts from a dense
prefill converted to the shallow form (both untimed).  Every kernel is
launched from Python through the C ABI; --graphs replays HIP graphs
captured from the same calls instead (one per run of step launches, one
per compression).

The metric is decode head-steps/s (whole job).  Also reported: the step
kernel's achieved HBM bandwidth from its algorithmic bytes and its average
launch duration (HIP events on the launch stream), the dense-state baseline
kernel on the same workload, two variants timed on the same state and
inputs -- the lazily decayed form (U's decay kept as a running product,
seed_decode_step_lazy) and the 16-bit form (kept factors fp16, rounded at
every compression, seed_decode_step_h16) -- staggered per-request
compression schedules (seed_decode_step_sched, one HIP graph), the handoff
of the converted
states (seed_pack_states / seed_unpack_states of every request), the
statistics of the prefilled states (seed_state_stats: sink energy share, top
direction, content ranks), and the CPU oracle timed on a bounded sample.
Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import torch  # noqa: E402

from sink_rank_recurrent_amd import binding  # noqa: E402
from sink_rank_recurrent_amd import workloads as wl  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor figure
DEFAULT_WORKLOAD = 2
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_seed_step_gdn_64x16_r16w32_bf16.json")
STEP_SOURCE = os.path.join(ROOT, "sink_rank_recurrent_amd", "csrc", "seed_step.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes (what the method must move; see the byte account in the
# design notes): reads a, r columns of U and V, the inputs and vbar; writes a,
# all r + 1 columns of U (in-place decay plus the new column), one V column
# and o (fp32).
# ---------------------------------------------------------------------------

def step_bytes_per_unit(w: wl.Workload, r: int, form: str = "in_place") -> float:
    """In place: U is read and written whole.  Lazy decay: U is only read,
    one new column is written, and the decay product (one float, or d_k for
    KDA) is read and written.  16-bit kept factors (lazy): the R kept
    columns are read at 2 bytes an entry, the r - R appended ones at 4."""
    s_in = 2 if w.in_dtype == torch.bfloat16 else 4
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


def dense_bytes_per_unit(w: wl.Workload) -> float:
    s_in = 2 if w.in_dtype == torch.bfloat16 else 4
    g_bytes = 4 * w.d_k if w.rule == "kda" else 4
    beta_bytes = 0 if w.rule == "mamba2" else 4
    return 8 * w.d_k * w.d_v + s_in * (2 * w.d_k + w.d_v) + g_bytes + beta_bytes + 4 * w.d_v


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(w: wl.Workload):
    """HBM bytes per step-kernel launch from the committed counter summary,
    or None if there is none or the kernel source changed since."""
    if w.name != wl.WORKLOADS[DEFAULT_WORKLOAD].name or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256_16") != source_hash(STEP_SOURCE):
        return None
    return t.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------

CONVERSION_MS = {}


def prepare(w: wl.Workload, layer: int, n_steps: int, dev: str, lazy: bool = False):
    """vbar, a converted shallow state and resident inputs for n_steps steps.
    The conversion (seed_state_from_dense of every head) is timed on the
    stream into CONVERSION_MS["ms"]."""
    vbar = wl.make_vbar(w.heads, w.d_v, w.seed, layer, dev)
    S = torch.zeros(w.batch, w.heads, w.d_k, w.d_v, device=dev)
    o = torch.empty(w.batch, w.heads, w.d_v, device=dev)
    for t in range(-w.prefill, 0):
        x = wl.workload_step(w, vbar, t, layer, dev)
        binding.dense_decode_step(w.rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)
    st = binding.ShallowState(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W, vbar, device=dev,
                              lazy=lazy)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st.from_dense(S)            # first call sets the kernel's LDS limit
    torch.cuda.synchronize()
    e0.record()
    st.from_dense(S)
    e1.record()
    inputs = [wl.workload_step(w, vbar, t, layer, dev) for t in range(n_steps)]
    torch.cuda.synchronize()
    CONVERSION_MS["ms"] = e0.elapsed_time(e1)
    return vbar, S, st, inputs


def _plan(st, warmup: int, steps: int):
    """The timed loop as a list of actions: ("steps", [(t, r), ...]) for each
    run of step launches between two compressions, ("compress", r) for each
    compression."""
    seq, cur, r = [], [], st.r
    for t in range(warmup, warmup + steps):
        cur.append((t, r))
        r += 1
        if r >= st.cap:
            seq.append(("steps", cur))
            cur = []
            seq.append(("compress", r))
            r = st.R
    if cur:
        seq.append(("steps", cur))
    return seq, r


def _do(st, step, inputs, o, action) -> None:
    """One action of the plan; `step` is the state's bound step call."""
    if action[0] == "steps":
        for t, r in action[1]:
            x = inputs[t]
            step(x["q"], x["k"], x["v"], x["g"], x["beta"], r)
    elif isinstance(st, binding.ShallowState16):
        binding.seed_compress_h16(st.rule, st.Uk, st.Vk, st.Uw, st.Vw, st.gam, action[1],
                                  st.rounding, st.seed, st.epoch)
        st.epoch += 1
    elif st.lazy:
        binding.seed_compress_lazy(st.rule, st.U, st.V, st.gam, action[1], st.R)
    else:
        binding.seed_compress(st.U, st.V, action[1], st.R)


def run_shallow(st, inputs, o, warmup: int, steps: int, graphs: bool):
    """Warm up eagerly, then time `steps` steps.

    With `graphs`, each run of step launches between two compressions and
    each compression is captured once as a HIP graph (untimed) and replayed
    in the timed loop, so host launch cost does not enter the timing.  HIP
    events on the launch stream bracket every action; no event marker sits
    between two step kernels."""
    for t in range(warmup):
        x = inputs[t]
        st.step_and_maybe_compress(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
    torch.cuda.synchronize()
    seq, r_end = _plan(st, warmup, steps)
    step = st.bind_step(o)
    captured = []
    if graphs:
        for action in seq:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                _do(st, step, inputs, o, action)
            captured.append(g)
        torch.cuda.synchronize()
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    marks = [ev() for _ in range(len(seq) + 1)]
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    for i, action in enumerate(seq):
        marks[i].record()
        if graphs:
            captured[i].replay()
        else:
            _do(st, step, inputs, o, action)
    marks[-1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    st.r = r_end
    windows, comp, step_r = [], [], []
    for i, action in enumerate(seq):
        ms = marks[i].elapsed_time(marks[i + 1])
        if action[0] == "steps":
            windows.append((ms, len(action[1])))
            step_r += [r for _, r in action[1]]
        else:
            comp.append(ms)
    return {
        "elapsed_s": marks[0].elapsed_time(marks[-1]) / 1e3,
        "wall_s": wall,
        "step_window_ms": windows,
        "step_r": step_r,
        "compress_ms": comp,
    }


def sched_bytes_per_unit(w: wl.Workload, r: int, D: int) -> float:
    """The lazy step's bytes at r columns, plus the merge step's fold of the
    decay product into the R + D held columns of U (once per W steps)."""
    return step_bytes_per_unit(w, r, "lazy") + 4 * w.d_k * (w.R + D) / w.W


def run_scheduled(w, S, vbar, inputs, warmup: int, steps: int, D: int, dev):
    """Staggered starts (request b's phase b mod W) on the per-request
    schedule with merge delay D, the snapshots of max(D, 1) consecutive
    steps compressed by one launch on the steps' stream.  Every request has
    passed its first merge when timing starts.  The timed steps and their
    compressions are captured once as one HIP graph and replayed."""
    t_start = [-(b % w.W) - (w.W + D) for b in range(w.batch)]
    st = binding.ScheduledState(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W, D, vbar,
                                t_start, device=dev)
    st.from_dense(S)
    o = torch.empty(w.batch, w.heads, w.d_v, device=dev)
    for t in range(warmup):
        x = inputs[t]
        st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
    st.join()
    torch.cuda.synchronize()
    # the columns every request holds at each timed step
    cols = [st.held_columns(b, t) for t in range(warmup, warmup + steps) for b in range(w.batch)]
    # every compression of the warm-up has finished: nothing to wait for
    st.pending.clear()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for t in range(warmup, warmup + steps):
            x = inputs[t]
            st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        st.join()
    torch.cuda.synchronize()
    st.pending.clear()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    el = e0.elapsed_time(e1) / 1e3
    units = w.batch * w.heads
    mean_bytes = sum(sched_bytes_per_unit(w, r, D) for r in cols) / len(cols)
    return {"D": D, "value": units * steps / el, "unit": "head-steps/s",
            "ms_per_step": el * 1e3 / steps, "mean_columns": sum(cols) / len(cols),
            "step_bytes_per_head_step": mean_bytes,
            "batch_steps": st.batch_steps, "side_streams": len(st.sides),
            "launch": "one hip graph of the timed steps; the snapshots of batch_steps "
                      "consecutive steps compressed by one launch on the steps' stream"}


def run_dense(w, S, inputs, o, warmup: int, steps: int, graphs: bool, chunk: int = 32):
    def do(ts):
        for t in ts:
            x = inputs[t]
            binding.dense_decode_step(w.rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)

    do(range(warmup))
    torch.cuda.synchronize()
    chunks = [range(c, min(c + chunk, warmup + steps)) for c in range(warmup, warmup + steps, chunk)]
    captured = []
    if graphs:
        for ts in chunks:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                do(ts)
            captured.append(g)
        torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i, ts in enumerate(chunks):
        if graphs:
            captured[i].replay()
        else:
            do(ts)
    t1.record()
    torch.cuda.synchronize()
    return {"elapsed_s": t0.elapsed_time(t1) / 1e3}


def _cpu_worker(job):
    """One host process of the CPU baseline: the oracle's factored mode, as it
    stands and on one thread, stepping its units through the inputs (cycled)
    and compressing every W, until the budget is spent."""
    rule, R, W, st0_np, inputs_np, budget_s = job
    from threadpoolctl import threadpool_limits

    import oracle

    a, U, V, vb = st0_np
    done = 0
    t0 = time.perf_counter()
    with threadpool_limits(limits=1):
        while time.perf_counter() - t0 < budget_s:
            x = inputs_np[done % len(inputs_np)]
            a, U, V, _ = oracle.seed_step(rule, a, U, V, vb, x["q"], x["k"], x["v"], x["g"],
                                          x["beta"])
            if U.shape[-1] >= R + W:
                U, V = oracle.compress(U, V, R)
            done += 1
    return a.shape[0], done, time.perf_counter() - t0


def cpu_baseline(w, st0_np, inputs_np, budget_s: float, workers: int):
    """The oracle on a bounded sample of the workload, on the host's cores:
    `workers` processes (spawned, so none inherits the GPU context), each
    with its own slice of the converted units and their inputs, all running
    for `budget_s` seconds at once.  The value is the sum of their rates."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor

    a, U, V, vb = st0_np
    n = a.shape[0]
    per = n // workers
    jobs = []
    for p in range(workers):
        sl = slice(p * per, (p + 1) * per)
        xs = [{k: (None if v is None else v[sl]) for k, v in x.items()} for x in inputs_np]
        jobs.append((w.rule, w.R, w.W, (a[sl], U[sl], V[sl], vb[sl]), xs, budget_s))
    with ProcessPoolExecutor(max_workers=workers,
                             mp_context=multiprocessing.get_context("spawn")) as ex:
        res = list(ex.map(_cpu_worker, jobs))
    rates = [units * done / el for units, done, el in res]
    steps = sum(done for _, done, _ in res)
    return {"value": sum(rates), "unit": "head-steps/s", "cores": workers, "kind": "oracle",
            "per_process": sum(rates) / workers,
            "sample": f"{workers} processes x {per} units, {steps} decode steps in all "
                      f"(compression every {w.W}) of {w.name}, from the converted state, "
                      f"fp64 numpy oracle, one thread per process, {budget_s:.0f} s each"}


def achievable_copy_GBs(n_bytes: int = 1 << 31, reps: int = 5) -> float:
    """Read + write GB/s of the library's streaming copy (seed_stream_copy)
    over a buffer far larger than the 256 MB memory-side cache: what HBM
    delivers to a read-once, write-once kernel here, set beside the nominal
    8 TB/s."""
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


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=sorted(wl.WORKLOADS))
    ap.add_argument("--layer", type=int, default=0)
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="host processes for the CPU baseline (default: the usable cores, "
                         "at most 16)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--lazy", action="store_true",
                    help="keep U's decay as a running product (seed_decode_step_lazy) instead of "
                         "rewriting U every step")
    ap.add_argument("--no-variant", action="store_true",
                    help="skip the lazily decayed and 16-bit forms that are otherwise timed as well")
    ap.add_argument("--graphs", action="store_true",
                    help="replay HIP graphs captured from the same calls instead of launching "
                         "every kernel from Python")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the shallow-state path has no cross-GPU exchange and "
              "this build runs on a single MI355X; --gpus must be 1", file=sys.stderr)
        return 2
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1

    if args.copy_probe:
        copy_probe()
        return 0

    w = wl.WORKLOADS[args.workload]
    steps = args.steps if args.steps is not None else min(w.steps, 1024)
    warmup = args.warmup
    dev = "cuda:0"
    torch.cuda.set_device(0)
    binding.lib()
    units = w.batch * w.heads
    log(f"workload {w.name}: {units} units, {steps} timed steps after {warmup} warm-up")

    vbar, S_dense, st, inputs = prepare(w, args.layer, warmup + steps, dev, lazy=args.lazy)
    log("prepared state and inputs")

    # snapshot for the CPU baseline (first units, converted state)
    cpu = None
    if not args.no_cpu:
        workers = args.cpu_workers or min(16, len(os.sched_getaffinity(0)))
        workers = max(1, min(workers, units // 16))
        n_cpu = min(units, 64 * workers) // workers * workers
        f64 = lambda t: t.detach().to("cpu", torch.float64).numpy()  # noqa: E731
        a0 = f64(st.a.reshape(units, w.d_k)[:n_cpu])
        U0 = f64(st.true_U().reshape(units, w.cap, w.d_k)[:n_cpu, :st.r]).transpose(0, 2, 1)
        V0 = f64(st.V.reshape(units, w.cap, w.d_v)[:n_cpu, :st.r]).transpose(0, 2, 1)
        vb0 = f64(vbar)[[u % w.heads for u in range(n_cpu)]]
        cpu_inputs = []
        for x in inputs[: min(len(inputs), 256)]:
            cpu_inputs.append({k: (None if v is None else f64(v.reshape((units,) + v.shape[2:])[:n_cpu]))
                               for k, v in x.items()})
        cpu_state = (a0, U0, V0, vb0)

    S_copy = S_dense.clone() if not args.no_dense else None
    S_var = S_dense.clone() if not (args.lazy or args.no_variant) else None
    o = torch.empty(w.batch, w.heads, w.d_v, device=dev)
    res = run_shallow(st, inputs, o, warmup, steps, graphs=args.graphs)
    log(f"shallow: {res['elapsed_s'] * 1e3:.2f} ms for {steps} steps")

    # the lazily decayed form and the 16-bit form on the same converted
    # state and inputs
    variants = {}
    if S_var is not None:
        for name, make, form in (
                ("lazy_decay_variant",
                 lambda: binding.ShallowState(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W,
                                              vbar, device=dev, lazy=True), "lazy"),
                ("fp16_factor_variant",
                 lambda: binding.ShallowState16(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W,
                                                vbar, store=torch.float16, rounding="nearest",
                                                device=dev), "h16")):
            st2 = make()
            st2.from_dense(S_var)
            r2 = run_shallow(st2, inputs, o, warmup, steps, graphs=args.graphs)
            s2 = sum(ms for ms, _ in r2["step_window_ms"]) / 1e3
            n2 = sum(n for _, n in r2["step_window_ms"])
            b2 = sum(step_bytes_per_unit(w, r, form) * units for r in r2["step_r"])
            variants[name] = {
                "value": units * steps / r2["elapsed_s"], "unit": "head-steps/s",
                "ms_per_step": r2["elapsed_s"] * 1e3 / steps,
                "step_bytes_per_head_step": b2 / n2 / units,
                "step_avg_launch_us": s2 / n2 * 1e6,
                "step_achieved_GBs": b2 / s2 / 1e9,
                "step_frac_of_peak": b2 / s2 / 1e9 / HBM_PEAK_GBS,
                "compress_avg_us": sum(r2["compress_ms"]) / max(1, len(r2["compress_ms"])) * 1e3}
            if form == "h16":
                variants[name]["factors"] = ("kept R columns fp16 (rounded to nearest at every "
                                             "compression), appended columns fp32, lazy decay")
            del st2
            log(f"{name}: {r2['elapsed_s'] * 1e3:.2f} ms for {steps} steps")
        del S_var

    # staggered per-request schedules: D = 0 (each compression finishes
    # before the next step) and a merge delay that hides it
    sched = None
    if not args.no_variant:
        sched = []
        # D = 0; the smallest delay whose batched launch fills every SIMD
        # once; half a window; the longest the ring allows
        cap_d = min(w.W - 1, 96 - w.R - w.W)
        simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count
        d_fill = min(cap_d, -(-simds // (units // w.W)))
        for D in sorted({0, d_fill, min(cap_d, w.W // 2), cap_d}):
            if w.R not in (16, 32):
                break
            sched.append(run_scheduled(w, S_dense, vbar, inputs, warmup, steps, D, dev))
            log(f"staggered schedule D={D}: {sched[-1]['ms_per_step'] * 1e3:.2f} us per step")

    # handoff of the converted states (prefill -> decode): pack every
    # request into one buffer, then unpack it into the slots of a batch
    handoff = None
    if not args.no_variant:
        hst = binding.ShallowState(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W, vbar,
                                   device=dev)
        hst.from_dense(S_dense)
        sel = torch.arange(w.batch, dtype=torch.int32, device=dev)
        buf = hst.pack(sel)
        reps = 20
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        ev[0].record()
        for _ in range(reps):
            hst.pack(sel, buf)
        ev[1].record()
        for _ in range(reps):
            hst.unpack(buf, sel)
        ev[2].record()
        torch.cuda.synchronize()
        nbytes = buf.numel()
        t_pack = ev[0].elapsed_time(ev[1]) / reps / 1e3
        t_unpack = ev[1].elapsed_time(ev[2]) / reps / 1e3
        handoff = {"head_bytes": nbytes // units, "dense_head_bytes": 4 * w.d_k * w.d_v,
                   "requests": w.batch, "buffer_bytes": nbytes,
                   "pack_us": t_pack * 1e6, "unpack_us": t_unpack * 1e6,
                   "pack_GBs": 2 * nbytes / t_pack / 1e9, "unpack_GBs": 2 * nbytes / t_unpack / 1e9}
        del hst, buf
        log(f"handoff: pack {t_pack * 1e6:.1f} us, unpack {t_unpack * 1e6:.1f} us for "
            f"{nbytes / 1e6:.1f} MB")

    # statistics of the converted workload's dense states (the quantities
    # the pages measure on model states), with the kernel's time
    stats = None
    if not args.no_variant:
        nf = binding.lib().seed_stat_fields()
        rec = torch.empty(w.batch, w.heads, nf, device=dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        binding.seed_state_stats(S_dense, vbar, w.R, rec)
        e1.record()
        torch.cuda.synchronize()
        r = rec.reshape(units, nf)[:, :len(binding.STAT_FIELDS)].double()
        med = {f: float(r[:, i].median()) for i, f in enumerate(binding.STAT_FIELDS)}
        stats = {"kernel_ms": e0.elapsed_time(e1), "units": units,
                 "median_sink_share": med["sink_share"], "median_top_share": med["top_share"],
                 "median_abs_cos_vstar_vbar": med["abs_cos_vstar_vbar"],
                 "median_rank90": med["rank90"], "median_rank99": med["rank99"],
                 "median_beyond_R_share": med["beyond_R_share"]}
        log(f"state statistics: {stats['kernel_ms']:.1f} ms for {units} heads")

    dense = None
    if not args.no_dense:
        dres = run_dense(w, S_copy, inputs, o, warmup, steps, graphs=args.graphs)
        d_bytes = dense_bytes_per_unit(w) * units
        d_avg = dres["elapsed_s"] / steps
        dense = {"value": units * steps / dres["elapsed_s"], "unit": "head-steps/s",
                 "bytes_per_head_step": dense_bytes_per_unit(w),
                 "kernel_avg_us": d_avg * 1e6,
                 "achieved_GBs": d_bytes / d_avg / 1e9}
        log(f"dense: {dres['elapsed_s'] * 1e3:.2f} ms")

    if not args.no_cpu:
        cpu = cpu_baseline(w, cpu_state, cpu_inputs, args.cpu_budget, workers)
        log(f"cpu oracle: {cpu['value']:.1f} head-steps/s on {workers} processes")

    elapsed = res["elapsed_s"]
    value = units * steps / elapsed
    step_total_s = sum(ms for ms, _ in res["step_window_ms"]) / 1e3
    comp_total_s = sum(res["compress_ms"]) / 1e3
    step_bytes = sum(step_bytes_per_unit(w, r, "lazy" if args.lazy else "in_place") * units
                     for r in res["step_r"])
    n_launch = sum(n for _, n in res["step_window_ms"])
    assert n_launch == len(res["step_r"])
    avg_launch_s = step_total_s / n_launch
    achieved = step_bytes / n_launch / avg_launch_s / 1e9
    copy_gbs = achievable_copy_GBs()
    log(f"plain 2 GiB device copy: {copy_gbs:.0f} GB/s read + write")
    traffic = None if args.lazy else load_traffic(w)
    mean_bytes = step_bytes / n_launch / units

    out = {
        "metric": "decode head-steps/s (sink + rank-R state update, whole job incl. compression)",
        "value": value,
        "unit": "head-steps/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": elapsed * 1e3 / steps,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded; no trace or checkpoint)",
        "config": {"workload": w.name, "rule": w.rule, "requests": w.batch, "heads": w.heads,
                   "layers_per_launch": 1, "d_k": w.d_k, "d_v": w.d_v, "R": w.R, "W": w.W,
                   "inputs": "bf16 q/k/v, fp32 gates" if w.in_dtype == torch.bfloat16 else "fp32",
                   "prefill": w.prefill,
                   "decay_of_U": "running product (lazy)" if args.lazy else "in place",
                   "launch": ("hip graphs (one per run of steps, one per compression)" if args.graphs
                              else "eager (one launch per kernel)")},
        "roofline": {"bound": "hbm", "kernel": "seed_step_kernel", "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic,
                     "algorithmic_bytes_per_launch": step_bytes / n_launch,
                     "avg_launch_us": avg_launch_s * 1e6,
                     "achievable_copy_GBs": copy_gbs,
                     "frac_of_achievable": achieved / copy_gbs if copy_gbs else None},
        "cpu_baseline": cpu,
        "breakdown": {"step_kernel_s": step_total_s, "compress_kernel_s": comp_total_s,
                      "compressions": len(res["compress_ms"]),
                      "compress_avg_us": (comp_total_s / max(1, len(res["compress_ms"]))) * 1e6,
                      "step_bytes_per_head_step": mean_bytes,
                      "step_only_head_steps_per_s": units * n_launch / step_total_s,
                      "wall_s": res["wall_s"]},
        "dense_baseline": dense,
        "lazy_decay_variant": variants.get("lazy_decay_variant"),
        "fp16_factor_variant": variants.get("fp16_factor_variant"),
        "conversion": {"kernel": "compress_wave_kernel (conversion instance)",
                       "ms": CONVERSION_MS.get("ms"), "heads": units,
                       "us_per_head": CONVERSION_MS.get("ms", 0.0) * 1e3 / units,
                       "what": "end-of-prefill sink split and rank-R truncation of every head "
                               "(C C^T by MFMA, Householder, multisection, inverse iteration; "
                               "once per request)"},
        "staggered_schedule_variants": sched,
        "handoff": handoff,
        "state_stats": stats,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
