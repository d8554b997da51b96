"""Whole-workload parity on the GPU at the benchmark's launch shapes.

Each workload runs exactly as bench.py runs it: a 512-step dense prefill
(dense_decode_step), the conversion to the shallow form
(seed_state_from_dense), then every decode step of the workload with a
compression whenever the window is full.  The 36-layer workload is checked
on three of its layers (0, 17 and 35), each at its full per-layer shape
(256 requests x 32 heads) over all 16384 decode steps, with the first
window bench.py gives it (W - floor(l W / L) steps: 32, 17 and 1), so the
staggered schedule is what is tested.

Two oracle runs follow sampled (request, head) units:
  * the oracle's own run: its own fp64 prefill, conversion, steps and
    compressions from the same seeded inputs, nothing taken from the GPU.
    Checked against it: the conversion (1e-4 relative, the two prefills
    differ by fp32 rounding); every read-out (1e-4); the state after every
    compression and at the last step (1e-4); and the sink coefficient `a`
    at EVERY step, across compressions, at 1e-5 -- by Lemma 1 (picx.dev
    summary, "Theoretical and Practical Implications") a follows its own
    d_k-vector recurrence that compression never touches;
  * a shadow run restarted from the GPU's own state after the conversion
    and after every compression, stepped on the identical inputs with no
    compression: the GPU's reconstructed state must stay within 1e-5 of it
    at every step until the next compression (Lemma 2's exactness between
    compressions).
A unit whose content has a near-tie at rank R ((s_R - s_{R+1}) / s_1 <
1e-4: the truncation is not unique) at its conversion or at any
compression is left out of the own-run checks from then on and counted;
at most 2 % of the compressions may be such.  Workloads 1-4 are also run in
the lazily decayed form (U = Diag(gam) U~), read back at true scale.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TIE_GAP, TOL_READOUT, TOL_STATE_COMPRESS, TOL_STATE_STEP, content_gap,
                      f64, rel_err, requires_gpu, state_rel_err, true_U)
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

TOL_SINK = 1e-5          # the sink coefficient a, every step (Lemma 1)


def _sample_units(total, k, seed):
    rng = np.random.default_rng(seed)
    picks = {0, total - 1}
    while len(picks) < min(k, total):
        picks.add(int(rng.integers(total)))
    return np.array(sorted(picks))


def _units_state(st, idx_t, r):
    """(a, U at true scale, V) of the sampled units, float64, math orientation."""
    cap = st.cap
    a = f64(st.a.reshape(-1, st.d_k)[idx_t])
    U = f64(true_U(st, idx_t)[:, :r]).transpose(0, 2, 1)
    V = f64(st.V.reshape(-1, cap, st.d_v)[idx_t, :r]).transpose(0, 2, 1)
    return a, U, V


def _units_inputs(x, idx_t):
    out = {}
    for key, t in x.items():
        if t is None:
            out[key] = None
        else:
            flat = t.reshape((-1,) + tuple(t.shape[2:]))
            out[key] = f64(flat[idx_t])
    return out


def first_window(w, layer):
    """bench.py's schedule: layer l's first window is W - floor(l W / L)."""
    return w.W - (layer * w.W) // w.layers


def run_workload(num, n_sample=8, steps=None, layer=0, lazy=False):
    w = wl.WORKLOADS[num]
    steps = w.steps if steps is None else steps
    dev = "cuda"
    units = w.batch * w.heads
    idx = _sample_units(units, n_sample, 77 + num + 1000 * layer)
    idx_t = torch.tensor(idx, device=dev)
    vbar = wl.make_vbar(w.heads, w.d_v, w.seed, layer, dev)
    vb = f64(vbar)[idx % w.heads]
    print(f"workload {num} layer {layer} lazy={lazy}: units {idx.tolist()}", flush=True)
    # dense prefill: the GPU for every unit, the oracle for the sampled ones
    S = torch.zeros(w.batch, w.heads, w.d_k, w.d_v, device=dev)
    o = torch.empty(w.batch, w.heads, w.d_v, device=dev)
    S_ref = np.zeros((len(idx), w.d_k, w.d_v))
    for t in range(-w.prefill, 0):
        x = wl.workload_step(w, vbar, t, layer, dev)
        binding.dense_decode_step(w.rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        S_ref, _ = oracle.dense_step(w.rule, S_ref, **_units_inputs(x, idx_t))
    st = binding.ShallowState(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W, vbar, device=dev,
                              lazy=lazy, first_window=first_window(w, layer))
    st.from_dense(S)
    torch.cuda.synchronize()
    a, U, V = oracle.state_from_dense(S_ref, vb, w.R)
    C = S_ref - a[..., :, None] * vb[..., None, :]
    ok = content_gap(C, np.broadcast_to(np.eye(w.d_v), C.shape[:-2] + (w.d_v, w.d_v)),
                     w.R) >= TIE_GAP
    stats = {"conversion": 0.0, "o": 0.0, "state": 0.0, "a": 0.0, "window": 0.0,
             "ties": int((~ok).sum()), "compressions": 0}
    ga, gU, gV = _units_state(st, idx_t, st.r)
    e_conv = state_rel_err(ga, gU, gV, a, U, V, vb)[ok]
    stats["conversion"] = float(e_conv.max()) if e_conv.size else 0.0
    assert stats["conversion"] < TOL_STATE_COMPRESS, e_conv
    sa, sU, sV = ga, gU, gV                      # the shadow run starts from the GPU's state

    for t in range(steps):
        x = wl.workload_step(w, vbar, t, layer, dev)
        st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        xi = _units_inputs(x, idx_t)
        a, U, V, o_ref = oracle.seed_step(w.rule, a, U, V, vb, **xi)
        sa, sU, sV, _ = oracle.seed_step(w.rule, sa, sU, sV, vb, **xi)
        ga, gU, gV = _units_state(st, idx_t, st.r)
        # Lemma 1: the sink coefficient against the oracle's own, every step
        e_a = rel_err(ga, a, -1)
        stats["a"] = max(stats["a"], float(e_a.max()))
        assert e_a.max() < TOL_SINK, (t, e_a)
        # Lemma 2: exact between compressions, from the GPU's own start
        e_w = state_rel_err(ga, gU, gV, sa, sU, sV, vb)
        stats["window"] = max(stats["window"], float(e_w.max()))
        assert e_w.max() < TOL_STATE_STEP, (t, e_w)
        e_o = rel_err(f64(o.reshape(-1, w.d_v)[idx_t]), o_ref, -1)[ok]
        if e_o.size:
            stats["o"] = max(stats["o"], float(e_o.max()))
            assert e_o.max() < TOL_READOUT, (t, e_o)
        last = t == steps - 1
        compressed = False
        if st.r >= st.limit:
            st.compress()
            compressed = True
            stats["compressions"] += 1
            tie = content_gap(U, V, w.R) < TIE_GAP
            stats["ties"] += int((tie & ok).sum())
            ok &= ~tie
            U, V = oracle.compress(U, V, w.R)
        if compressed or last:
            ga, gU, gV = _units_state(st, idx_t, st.r)
            sa, sU, sV = ga, gU, gV
            if ok.any():
                e_s = state_rel_err(ga, gU, gV, a, U, V, vb)[ok]
                stats["state"] = max(stats["state"], float(e_s.max()))
                assert e_s.max() < TOL_STATE_COMPRESS, (t, e_s)
    n_checks = len(idx) * (1 + stats["compressions"])
    assert stats["ties"] <= max(1, n_checks // 50), stats
    assert ok.sum() >= len(idx) // 2, stats
    return stats


@pytest.mark.parametrize("num", [1, 2, 3, 4])
def test_workload_parity(num):
    n_sample = 1 if num == 1 else 8
    stats = run_workload(num, n_sample=n_sample)
    print(f"workload {num}: {stats}")


@pytest.mark.parametrize("layer", [0, 17, 35])
def test_workload5_layer_parity(layer):
    """Three layers of the 36-layer workload, each at its own compression
    phase, over all 16384 steps."""
    stats = run_workload(5, n_sample=6, layer=layer)
    assert stats["compressions"] == 1 + (16384 - first_window(wl.WORKLOADS[5], layer)) // 32
    print(f"workload 5, layer {layer}: {stats}")


@pytest.mark.parametrize("num", [1, 2, 3, 4])
def test_workload_parity_lazy_decay(num):
    """The same checks on the lazily decayed form (seed_decode_step_lazy /
    seed_compress_lazy), its state read at true scale, U = Diag(gam) U~."""
    stats = run_workload(num, n_sample=1 if num == 1 else 6, lazy=True)
    print(f"workload {num}, lazy decay: {stats}")


def test_workload5_layer_parity_lazy_decay():
    """The lazily decayed form on the 36-layer workload's middle layer over
    all 16384 steps (the form bench.py reports first)."""
    stats = run_workload(5, n_sample=6, layer=17, lazy=True)
    assert stats["compressions"] == 1 + (16384 - first_window(wl.WORKLOADS[5], 17)) // 32
    print(f"workload 5, layer 17, lazy decay: {stats}")
