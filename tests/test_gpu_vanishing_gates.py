"""The lazily decayed forms with gates that drive the running decay product
to nothing within a window (see include/seed.h, seed_decode_step_lazy): a
product below 2^-64 is folded into the held columns and restarted, so the
state keeps following Lemma 2.

Gates are drawn from 5e-3 .. 2e-2 for Gated DeltaNet and Mamba-2 (the
product of a window of 32 such gates is about 1e-64, far below the normal
fp32 range), and per channel from 5e-3 .. 0.999 for Kimi Delta Attention,
so that some channels fold and others do not.  Each form runs a window of
W steps and a compression from the same start as the oracle, which runs on
its own (in place, fp64): every read-out within 1e-4, the state within 1e-5
at every step and within 1e-4 after the compression (relative, per unit),
and no value may be NaN or infinite.  The 16-bit form with fp16 kept
factors is checked the same way (its kept columns fold to zero once their
product is below 2^-64); the per-request schedule is run with D = 0 and
with a merge delay over several windows.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TIE_GAP, TOL_READOUT, TOL_STATE_COMPRESS, TOL_STATE_STEP, f64, inputs_np,
                      rel_err, requires_gpu, sched_true_factors, state_rel_err, true_factors16,
                      true_U)
from oracle import seed_schedule as sc
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

B, H = 3, 4


def _small_gates(rule, x, gen):
    g = x["g"]
    if rule == "kda":
        lo = torch.where(torch.rand(g.shape, device="cuda", generator=gen) < 0.5, 5e-3, 0.9)
        hi = torch.where(lo < 0.5, 2e-2, 0.999)
    else:
        lo, hi = 5e-3, 2e-2
    x["g"] = (lo + (hi - lo) * torch.rand(g.shape, device="cuda", generator=gen)).contiguous()
    return x


def _start(rule, d_k, d_v, R, gen):
    vbar = torch.randn(H, d_v, device="cuda", generator=gen)
    a0 = torch.randn(B, H, d_k, device="cuda", generator=gen)
    U0 = torch.linalg.qr(torch.randn(B, H, d_k, R, device="cuda", generator=gen))[0]
    V0 = torch.randn(B, H, R, d_v, device="cuda", generator=gen)
    return vbar, a0, U0.transpose(-1, -2).contiguous(), V0


def _oracle_start(vbar, a0, U0, V0, d_v):
    vb = np.broadcast_to(f64(vbar)[None], (B, H, d_v)).reshape(-1, d_v)
    a = f64(a0).reshape(B * H, -1)
    U = f64(U0).reshape(B * H, U0.shape[2], -1).transpose(0, 2, 1)
    V = f64(V0).reshape(B * H, V0.shape[2], -1).transpose(0, 2, 1)
    return a, U, V, vb


def _finite(*ts):
    return all(bool(torch.isfinite(t).all()) for t in ts)


@pytest.mark.parametrize("form", ["lazy", "fp16", "bf16"])
@pytest.mark.parametrize("rule,dims,R,W", [("gdn", (128, 128), 16, 32), ("kda", (128, 128), 16, 32),
                                           ("mamba2", (128, 64), 16, 32), ("gdn", (64, 64), 16, 24)])
def test_fold_keeps_lemma2(form, rule, dims, R, W):
    d_k, d_v = dims
    gen = torch.Generator(device="cuda").manual_seed(301)
    vbar, a0, U0, V0 = _start(rule, d_k, d_v, R, gen)
    if form == "lazy":
        st = binding.ShallowState(rule, B, H, d_k, d_v, R, W, vbar, device="cuda", lazy=True)
        st.U[:, :, :R] = U0
        st.V[:, :, :R] = V0
    else:
        store = torch.float16 if form == "fp16" else torch.bfloat16
        st = binding.ShallowState16(rule, B, H, d_k, d_v, R, W, vbar, store=store, device="cuda")
        st.Uk.copy_(U0.to(store))
        st.Vk.copy_(V0.to(store))
        U0, V0 = st.Uk.float(), st.Vk.float()      # the oracle starts from the stored values
    st.a.copy_(a0)
    st.r = R
    a, U, V, vb = _oracle_start(vbar, a0, U0, V0, d_v)
    o = torch.empty(B, H, d_v, device="cuda")
    folded = False
    for t in range(W):
        x = _small_gates(rule, wl.make_step(rule, B, H, d_k, d_v, vbar, 302, t, 0, torch.bfloat16,
                                            "cuda"), gen)
        st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        a, U, V, o_ref = oracle.seed_step(rule, a, U, V, vb, **inputs_np(x))
        if form == "lazy":
            gU = true_U(st)[:, :, :st.r]
            gV = st.V[:, :, :st.r]
        else:
            gU, gV = true_factors16(st)
        assert _finite(o, st.a, gU, gV, st.gam), t
        folded = folded or bool((st.gam == 1.0).any()) and t > 0
        assert float(st.gam.min()) >= 2.0 ** -64 * 5e-3, t
        ga = f64(st.a).reshape(B * H, -1)
        gUn = f64(gU).reshape(B * H, st.r, -1).transpose(0, 2, 1)
        gVn = f64(gV).reshape(B * H, st.r, -1).transpose(0, 2, 1)
        assert rel_err(f64(o).reshape(-1, d_v), o_ref, -1).max() < TOL_READOUT, t
        assert state_rel_err(ga, gUn, gVn, a, U, V, vb).max() < TOL_STATE_STEP, t
    assert folded, "no decay product was folded: the test does not reach the guarded case"
    st.compress()
    torch.cuda.synchronize()
    U, V = oracle.compress(U, V, R)
    if form == "lazy":
        gU, gV = true_U(st)[:, :, :R], st.V[:, :, :R]
    else:
        gU, gV = true_factors16(st)
    ga = f64(st.a).reshape(B * H, -1)
    gUn = f64(gU).reshape(B * H, R, -1).transpose(0, 2, 1)
    gVn = f64(gV).reshape(B * H, R, -1).transpose(0, 2, 1)
    # the 16-bit forms round the kept factors once: 4u of the stored format
    tol = TOL_STATE_COMPRESS if form == "lazy" else (4 * 2.0 ** -11 if form == "fp16" else 4 * 2.0 ** -8)
    assert state_rel_err(ga, gUn, gVn, a, U, V, vb).max() < tol


@pytest.mark.parametrize("D", [0, 6])
@pytest.mark.parametrize("rule", ["gdn", "kda"])
def test_fold_in_per_request_schedule(rule, D):
    """Staggered requests over three windows with vanishing gates: every
    read-out and the final states follow the oracle's own schedule run
    (each unit from the same converted state, on its own).  Kimi Delta
    Attention's slow channels keep content of full rank in their subspace,
    so a snapshot can hold a near-tie at rank R whose trailing singular
    value is not negligible (s_{R+1} above 1e-5 s_1: a truncation that is
    not unique to within the tolerance); as in the other schedule tests, the
    first such snapshot of a unit ends its comparison, and at most a quarter
    of the units may end early.  Where s_{R+1} is below that, every
    truncation is as good and the comparison goes on."""
    d_k, d_v, R, W = 128, 128, 16, 16
    gen = torch.Generator(device="cuda").manual_seed(303)
    vbar = torch.randn(H, d_v, device="cuda", generator=gen)
    vb = f64(vbar)
    t_start = [0, 3, 11][:B]
    T = max(t_start) + 3 * W + D + 2
    rng = np.random.default_rng(304)
    vbu = np.broadcast_to(vb[None], (B, H, d_v)).reshape(-1, d_v)
    a0, U0, V0 = oracle.state_from_dense(0.1 * rng.standard_normal((B * H, d_k, d_v)), vbu, R)
    a0, U0, V0 = (x.astype(np.float32).astype(np.float64) for x in (a0, U0, V0))
    st = binding.ScheduledState(rule, B, H, d_k, d_v, R, W, D, vbar, t_start, device="cuda")
    st.a.copy_(torch.tensor(a0.reshape(B, H, d_k), dtype=torch.float32))
    st.KU[0].copy_(torch.tensor(U0.transpose(0, 2, 1).reshape(B, H, R, d_k), dtype=torch.float32))
    st.KV[0].copy_(torch.tensor(V0.transpose(0, 2, 1).reshape(B, H, R, d_v), dtype=torch.float32))
    xs = [_small_gates(rule, wl.make_step(rule, B, H, d_k, d_v, vbar, 305, t, 0, torch.bfloat16,
                                          "cuda"), gen) for t in range(T)]
    o = torch.empty(B, H, d_v, device="cuda")
    outs = []
    for t in range(T):
        st.step(xs[t]["q"], xs[t]["k"], xs[t]["v"], xs[t]["g"], xs[t]["beta"], o)
        outs.append(o.clone())
    st.join()
    torch.cuda.synchronize()
    assert _finite(st.gam, *outs)
    outs = [f64(x) for x in outs]
    skipped = 0
    for u in range(B * H):
        b, h = divmod(u, H)
        t0 = t_start[b]
        steps = [{k: (None if v is None else f64(v[b, h])) for k, v in xs[t].items()}
                 for t in range(t0, T)]
        a, U, V, o_ref, ev = sc.scheduled_run(rule, a0[u], U0[u], V0[u], vb[h], steps, R, W, D)
        gaps = [(e[0], e[2], e[3]) for e in ev if e[1] == "snapshot"]
        bad = [A for A, gap, tail in gaps if gap < TIE_GAP and tail > 1e-5]
        last = t0 + (bad[0] if bad else len(steps))
        skipped += bool(bad)
        for t in range(t0, last):
            assert rel_err(outs[t][b, h], o_ref[t - t0], -1) < TOL_READOUT, (u, t, gaps)
        if bad:
            continue
        gU, gV = sched_true_factors(st, b, h)
        Sg = oracle.reconstruct(f64(st.a[b, h]), f64(gU), f64(gV), vb[h])
        Sr = oracle.reconstruct(a, U, V, vb[h])
        assert rel_err(Sg, Sr, (-2, -1)) < TOL_STATE_COMPRESS, u
    assert skipped <= B * H // 4, skipped
