"""Per-request schedules (seed_decode_step_sched / seed_compress_sched, the
binding's ScheduledState) on the GPU against the oracle's schedule
(oracle/seed_schedule.py), each unit from the same converted state on the
same inputs, the oracle running its own schedule from its own conversion.

Requests start at different steps (one starts late, so it idles first).
Bars: every read-out of a started request to 1e-4 relative, an idle
request's read-out exactly zero; states at checkpoints to 1e-4 relative
(they follow compressions).  A unit whose snapshot content has a near-tie
at rank R ((s_R - s_{R+1})/s_1 < 1e-4: the truncation is not unique) is
left out from that snapshot on and counted."""
import numpy as np
import pytest
import torch

from gpu_util import (TIE_GAP, TOL_READOUT, TOL_STATE_COMPRESS, f64, rel_err, requires_gpu,
                      sched_true_factors)
from oracle import seed_oracle as so
from oracle import seed_schedule as sc
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs_of(x, u, H):
    b, h = divmod(u, H)
    return {k: (None if v is None else f64(v[b, h])) for k, v in x.items()}


@pytest.mark.parametrize("rule,dims,W,D,K,NS,R", [
    ("gdn", (128, 128), 16, 0, 1, 0, 16), ("gdn", (128, 128), 16, 6, None, 0, 16),
    ("kda", (128, 128), 32, 12, 5, 3, 16), ("mamba2", (128, 64), 16, 5, 3, 1, 16),
    ("gdn", (64, 64), 16, 15, None, 2, 16), ("kda", (128, 128), 32, 8, None, 0, 32)])
def test_scheduled_run_matches_oracle(rule, dims, W, D, K, NS, R):
    """K: the snapshots of K consecutive steps share one compression launch
    (None: the default, max(D, 1)); NS: side streams the launches alternate
    over (0: in order on the steps' stream); R: 16 or 32 kept columns."""
    d_k, d_v = dims
    B, H = 5, 3
    t_start = [0, 1, 4, 9, 2 * W + 3]
    T = max(t_start) + 2 * W + D + 3
    seed = 900 + W + D
    vbar = wl.make_vbar(H, d_v, seed, 0, "cpu")
    vb = f64(vbar)
    # the converted states: the oracle's conversion of dense states it
    # prefilled itself, stored as the GPU's initial state
    S = np.zeros((B * H, d_k, d_v))
    for t in range(-48, 0):
        x = wl.make_step(rule, B, H, d_k, d_v, vbar, seed, t, 0, torch.bfloat16, "cpu")
        xi = {k: (None if v is None else f64(v).reshape((B * H,) + tuple(v.shape[2:])))
              for k, v in x.items()}
        S, _ = so.dense_step(rule, S, **xi)
    vbu = np.broadcast_to(vb[None], (B, H, d_v)).reshape(-1, d_v)
    a0, U0, V0 = so.state_from_dense(S, vbu, R)
    a0, U0, V0 = (x.astype(np.float32).astype(np.float64) for x in (a0, U0, V0))
    st = binding.ScheduledState(rule, B, H, d_k, d_v, R, W, D, vbar.cuda(), t_start,
                                batch_steps=K, side_streams=NS)
    st.a.copy_(torch.tensor(a0.reshape(B, H, d_k), dtype=torch.float32))
    st.KU[0].copy_(torch.tensor(U0.transpose(0, 2, 1).reshape(B, H, R, d_k), dtype=torch.float32))
    st.KV[0].copy_(torch.tensor(V0.transpose(0, 2, 1).reshape(B, H, R, d_v), dtype=torch.float32))

    xs = [wl.make_step(rule, B, H, d_k, d_v, vbar, seed + 1, t, 0, torch.bfloat16, "cuda")
          for t in range(T)]
    o = torch.empty(B, H, d_v, device="cuda")
    outs = []
    checkpoints = {T // 2, T - 1}
    gpu_states = {}
    for t in range(T):
        st.step(xs[t]["q"], xs[t]["k"], xs[t]["v"], xs[t]["g"], xs[t]["beta"], o)
        outs.append(o.clone())
        if t in checkpoints:
            st.join()
            torch.cuda.synchronize()
            gpu_states[t] = {(b, h): [f64(m) for m in sched_true_factors(st, b, h)] + [f64(st.a[b, h])]
                             for b in range(B) for h in range(H)}
    st.join()
    torch.cuda.synchronize()
    outs = [f64(x) for x in outs]

    skipped = 0
    for u in range(B * H):
        b, h = divmod(u, H)
        t0 = t_start[b]
        steps = [_inputs_of(xs[t], u, H) for t in range(t0, T)]
        a, U, V, o_ref, ev = sc.scheduled_run(rule, a0[u], U0[u], V0[u], vb[h], steps, R, W, D)
        # the first snapshot whose truncation is not unique ends the comparison
        bad = [A for A, kind, *gap in ev if kind == "snapshot" and gap[0] < TIE_GAP]
        last = t0 + (bad[0] if bad else len(steps))
        skipped += bool(bad)
        for t in range(T):
            if t < t0:
                assert np.all(outs[t][b, h] == 0.0), (u, t)
            elif t < last:
                assert rel_err(outs[t][b, h], o_ref[t - t0], -1) < TOL_READOUT, (u, t)
        for tc, states in gpu_states.items():
            n = tc + 1 - t0
            if n <= 0 or tc >= last:
                continue
            ra, rU, rV, _, _ = sc.scheduled_run(rule, a0[u], U0[u], V0[u], vb[h], steps[:n], R, W,
                                                D)
            gU, gV, ga = states[(b, h)]
            assert gU.shape[1] == rU.shape[1] == sc.columns_before_step(n, R, W, D), (u, tc)
            Sg = so.reconstruct(ga, gU, gV, vb[h])
            Sr = so.reconstruct(ra, rU, rV, vb[h])
            assert rel_err(Sg, Sr, (-2, -1)) < TOL_STATE_COMPRESS, (u, tc)
    assert skipped <= B * H // 4, skipped


@pytest.mark.parametrize("num,D", [(2, 16), (5, 8), (5, 2)])
def test_scheduled_launch_size_sampled(num, D):
    """Launch-size per-request schedules with starts spread over the W
    phases, sampled heads against the oracle's schedule from the oracle's
    own conversion of its own prefill: workload 2 (64 requests x 16 GDN
    heads, R = 16, W = 32) at D = 16, and one layer of the 36-layer
    workload (256 requests x 32 heads, 8192 units, the 256-thread step
    workgroup) at D = 8 (up to 55 held columns) and at D = 2, as bench.py
    times it."""
    w = wl.WORKLOADS[num]
    B, H, R, W = w.batch, w.heads, w.R, w.W
    units = B * H
    t_start = [b % W for b in range(B)]
    idx = np.array([0, 17, 330, 700, units - 1] if num == 2 else [0, 17, 2731, 5466, units - 1])
    vbar = wl.make_vbar(H, w.d_v, w.seed, 0, "cuda")
    vb = f64(vbar)[idx % H]
    S = torch.zeros(B, H, w.d_k, w.d_v, device="cuda")
    o = torch.empty(B, H, w.d_v, device="cuda")
    S_ref = np.zeros((len(idx), w.d_k, w.d_v))

    def sample(x):
        return {k: (None if v is None else f64(v.reshape((units,) + tuple(v.shape[2:]))[idx]))
                for k, v in x.items()}

    for t in range(-64, 0):
        x = wl.workload_step(w, vbar, t, 0, "cuda")
        binding.dense_decode_step(w.rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        S_ref, _ = so.dense_step(w.rule, S_ref, **sample(x))
    st = binding.ScheduledState(w.rule, B, H, w.d_k, w.d_v, R, W, D, vbar, t_start)
    st.from_dense(S)
    a0, U0, V0 = so.state_from_dense(S_ref, vb, R)
    T = W - 1 + 2 * W + D + 2
    xs = []
    outs = []
    for t in range(T):
        x = wl.workload_step(w, vbar, t, 0, "cuda")
        xs.append(sample(x))
        st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        outs.append(f64(o.reshape(units, w.d_v)[idx]))
    st.join()
    torch.cuda.synchronize()
    skipped = 0
    for i, u in enumerate(idx):
        b = u // H
        t0 = t_start[b]
        steps = [{k: (None if v is None else v[i]) for k, v in xs[t].items()}
                 for t in range(t0, T)]
        _, _, _, o_ref, ev = sc.scheduled_run(w.rule, a0[i], U0[i], V0[i], vb[i], steps, R, W, D)
        bad = [A for A, kind, *gap in ev if kind == "snapshot" and gap[0] < TIE_GAP]
        last = t0 + (bad[0] if bad else len(steps))
        skipped += bool(bad)
        for t in range(T):
            if t < t0:
                assert np.all(outs[t][i] == 0.0), (u, t)
            elif t < last:
                # the conversions differ by the prefill's fp32 rounding
                assert rel_err(outs[t][i], o_ref[t - t0], -1) < TOL_READOUT, (u, t)
    assert skipped <= 1
