"""bench.py's host side without a GPU: the one-GPU rule and the algorithmic
byte account the roofline divides by."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sink_rank_recurrent_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def _mean(w, form):
    rs = range(w.R, w.R + w.W)          # columns held before each step of a window
    sp = bench.Spec(w)
    return sum(bench.step_bytes_per_unit(sp, r, form) for r in rs) / w.W


def test_step_bytes_per_head_step_workload2():
    """Workload 2 (GDN 128 x 128, bf16 q/k/v, R = 16, W = 32, 64 requests):
    the per-head-step bytes of each form, mean r = 31.5."""
    w = wl.WORKLOADS[2]
    sp = bench.Spec(w)
    assert _mean(w, "in_place") == pytest.approx(51728.0)
    assert _mean(w, "lazy") == pytest.approx(35608.0)
    assert _mean(w, "h16") == pytest.approx(27416.0)
    # the dense baseline reads and writes the whole state
    assert bench.dense_bytes_per_unit(sp) == 8 * 128 * 128 + 2 * (2 * 128 + 128) + 4 + 4 + 4 * 128


def test_byte_account_terms():
    """Each term of the account, at one r: factors read (and U written in
    place), the appended columns, a, the inputs, the gates, vbar's share."""
    w = bench.Spec(wl.WORKLOADS[3])            # Mamba-2 128 x 64, no beta, 128 requests
    r = 20
    d_k, d_v = w.d_k, w.d_v
    read = 4 * d_k + 4 * (d_k + d_v) * r + 2 * (2 * d_k + d_v) + 4 + 4 * d_v / w.batch
    write_in_place = 4 * d_k + 4 * d_k * (r + 1) + 4 * d_v + 4 * d_v
    assert bench.step_bytes_per_unit(w, r, "in_place") == pytest.approx(read + write_in_place)
    lazy = read + 4 + 4 * d_k + 4 * d_k + 4 * d_v + 4 * d_v + 4
    assert bench.step_bytes_per_unit(w, r, "lazy") == pytest.approx(lazy)
    h16 = lazy - 2 * (d_k + d_v) * w.R
    assert bench.step_bytes_per_unit(w, r, "h16") == pytest.approx(h16)


class _St:
    """Host bookkeeping of a layer's state, as bench.plan reads it."""

    def __init__(self, R, W, first_window):
        self.R, self.W, self.cap = R, W, R + W
        self.r, self.limit = R, R + first_window


def test_layer_phases_spread_compressions():
    """36 layers, W = 32: the first windows W - phase cover every length
    1..32 at most twice, and over any K consecutive steps after the first
    window the compressions are L K / W to within the layers per phase."""
    L, W, R = 36, 32, 16
    ph = bench.layer_phases(L, W)
    assert ph[0] == 0 and max(ph) == W - 1 and sorted(ph) == ph
    assert max(ph.count(p) for p in range(W)) == 2
    states = [_St(R, W, W - p) for p in ph]
    pl, r_end, lim_end = bench.plan(states, 5 * W)
    # every layer steps every bench step, and compresses every W steps
    for steps, comps in pl:
        assert [l for l, _ in steps] == list(range(L))
    per_layer = [[i for i, (_, comps) in enumerate(pl) if any(l == m for m, _ in comps)]
                 for l in range(L)]
    for l, idx in enumerate(per_layer):
        assert idx[0] == W - ph[l] - 1
        assert all(b - a == W for a, b in zip(idx, idx[1:]))
    for K in (1, 5, 20, 32, 64):
        for t0 in range(W, 3 * W):
            n = sum(len(c) for _, c in pl[t0:t0 + K])
            assert abs(n - L * K / W) <= 2, (K, t0, n)
    # the columns a step sees never exceed the capacity; compressions take r = limit
    for steps, comps in pl:
        assert all(states[l].R <= r < states[l].cap for l, r in steps)
    # plan leaves the states untouched
    assert all(st.r == R for st in states)


def test_cpu_worker_and_no_leftover_process(tmp_path):
    """The CPU baseline's oracle processes: each runs the factored and the
    dense oracle on its slice and is waited for, so no child outlives the
    call."""
    import numpy as np
    import psutil

    import oracle

    rng = np.random.default_rng(5)
    n, d_k, d_v, R, W = 4, 8, 8, 2, 3
    vb = rng.standard_normal((n, d_v))
    S = rng.standard_normal((n, d_k, d_v))
    a, U, V = oracle.state_from_dense(S, vb, R)
    xs = []
    for _ in range(4):
        k = rng.standard_normal((n, d_k))
        q = rng.standard_normal((n, d_k))
        xs.append({"q": q / np.linalg.norm(q, axis=-1, keepdims=True),
                   "k": k / np.linalg.norm(k, axis=-1, keepdims=True),
                   "v": vb + 0.3 * rng.standard_normal((n, d_v)),
                   "g": rng.uniform(0.9, 0.999, n), "beta": rng.uniform(0, 1, n)})

    Sp = type("Sp", (), {"rule": "gdn", "R": R, "W": W, "name": "tiny"})

    before = {c.pid for c in psutil.Process().children(recursive=True)}
    res = bench.cpu_baseline(Sp, (a, U, V, vb, S, xs), 0.5, 0.2, 2)
    after = {c.pid for c in psutil.Process().children(recursive=True)}
    assert after <= before
    assert res["cores"] == 2 and res["value"] > 0 and res["dense_value"] > 0
    assert res["single_thread_value"] == pytest.approx(res["value"] / 2)
    assert res["host_cpus_usable"] >= 1


def test_ops_group_step_runs():
    """Sequential: consecutive step launches with no compression between
    them form one graph, the compressions of a bench step follow its L
    launches.  Overlapped: a layer's compression is forked right after the
    step launch that ends its window and waited for right before that
    layer's next step launch, with the other L - 1 layers' launches between.
    Every launch appears once, in order, in both."""
    L, W, R = 36, 32, 16
    ph = bench.layer_phases(L, W)
    pl, _, _ = bench.plan([_St(R, W, W - p) for p in ph], 40)
    ops = bench._ops(pl, 5, 25, False, set())
    launches = [(t, l) for op in ops if op[0] == "steps" for t, l, _ in op[1]]
    assert launches == [(t, l) for t in range(5, 25) for l in range(L)]
    comps = [c for op in ops if op[0] == "compress" for c in op[1]]
    assert comps == [c for t in range(5, 25) for c in pl[t][1]]
    assert all(a[0] != b[0] for a, b in zip(ops, ops[1:]))
    # one layer: a whole window of W steps is one run
    pl1, _, _ = bench.plan([_St(R, W, W)], 3 * W)
    ops1 = bench._ops(pl1, W, 3 * W, False, set())
    assert [(op[0], len(op[1])) for op in ops1] == [("steps", W), ("compress", 1)] * 2

    pending = set()
    ops = bench._ops(pl, 5, 25, True, pending)
    seq = []
    for op in ops:
        if op[0] == "steps":
            seq += [("step", t, l) for t, l, _ in op[1]]
        else:
            seq.append(op)
    assert [(x[1], x[2]) for x in seq if x[0] == "step"] == \
        [(t, l) for t in range(5, 25) for l in range(L)]
    forks = [(i, x) for i, x in enumerate(seq) if x[0] == "fork"]
    assert [(x[1], x[2]) for _, x in forks] == [c for t in range(5, 25) for c in pl[t][1]]
    for i, (_, l, r) in forks:
        # right after the step of layer l that ends its window
        assert seq[i - 1][0] == "step" and seq[i - 1][2] == l
        nxt = [j for j in range(i + 1, len(seq)) if seq[j][0] == "step" and seq[j][2] == l]
        if nxt:
            j = nxt[0]
            assert seq[j - 1] == ("wait", l)
            assert sum(1 for x in seq[i:j] if x[0] == "step") == L - 1
        else:
            assert l in pending
    assert sum(1 for x in seq if x[0] == "wait") + len(pending) == len(forks)


@pytest.mark.parametrize("num, cols", [(5, 48), (4, 80)])
def test_compression_counters_parse(num, cols):
    """The committed compression counters give the MFMA work per unit that
    the compression roofline divides: MOPS x 512 agrees with the MFMA
    instruction count x 2048 flops of v_mfma_f32_16x16x4f32 (each summary
    rounds to four digits), and the bytes per unit are those of n = R + W
    columns read and R written."""
    w = wl.WORKLOADS[num]
    c = bench.load_compress_counters(w)
    assert c is not None, bench.counters_file(w)
    assert abs(c["mfma_flops_per_unit"] / (c["mfma_insts_per_unit"] * 2048) - 1) < 1e-3
    rec = bench.compression_roofline(w, 1000, 100.0)
    assert rec["columns"] == cols
    assert rec["bytes_per_unit"] == 4 * (w.d_k + w.d_v) * (cols + w.R)
    assert abs(rec["mfma_achieved_TFLOPs"] - c["mfma_flops_per_unit"] * 1000 / 1e-4 / 1e12) < 1e-9
    assert bench.compression_roofline(w, 1000, None) is None
