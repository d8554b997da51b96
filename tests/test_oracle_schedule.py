"""Pins of the per-request schedule oracle (oracle/seed_schedule.py)."""
import numpy as np
import pytest

from oracle import seed_oracle as so
from oracle import seed_schedule as sc


def _steps(rule, rng, n, d_k, d_v, vbar):
    out = []
    for _ in range(n):
        k = rng.standard_normal(d_k)
        k /= np.linalg.norm(k)
        q = rng.standard_normal(d_k)
        q /= np.linalg.norm(q)
        x = {"q": q, "k": k, "v": vbar + 0.3 * rng.standard_normal(d_v)}
        if rule == "kda":
            x["g"] = rng.uniform(0.9, 1.0, d_k)
        else:
            x["g"] = rng.uniform(0.9, 1.0)
        x["beta"] = None if rule == "mamba2" else rng.uniform(0, 1)
        out.append(x)
    return out


@pytest.mark.parametrize("rule", ["gdn", "kda", "mamba2"])
def test_no_delay_is_the_factored_run(rule):
    """D = 0 compresses at the snapshot: the aligned reading per request."""
    rng = np.random.default_rng(1)
    d_k, d_v, R, W = 12, 10, 3, 4
    vbar = rng.standard_normal(d_v)
    S = rng.standard_normal((d_k, d_v))
    a, U, V = so.state_from_dense(S, vbar, R)
    steps = _steps(rule, rng, 3 * W + 2, d_k, d_v, vbar)
    a1, U1, V1, o1, ev = sc.scheduled_run(rule, a, U, V, vbar, steps, R, W, 0)
    a2, U2, V2, o2 = so.factored_run(rule, a, U, V, vbar, steps, R, W)
    assert np.allclose(np.array(o1), np.array(o2), atol=1e-12)
    assert np.allclose(U1 @ V1.T, U2 @ V2.T, atol=1e-12) and np.allclose(a1, a2)
    assert [e for e in ev if e[1] == "merge"] == [(W, "merge"), (2 * W, "merge"), (3 * W, "merge")]


@pytest.mark.parametrize("rule", ["gdn", "kda", "mamba2"])
@pytest.mark.parametrize("D", [0, 1, 3])
def test_full_rank_reproduces_the_dense_recurrence(rule, D):
    """With R = min(d_k, d_v) every truncation is exact, so any delay gives
    the dense run's read-outs and state."""
    rng = np.random.default_rng(2)
    d_k, d_v, W = 5, 4, 4
    R = 4
    vbar = rng.standard_normal(d_v)
    S = rng.standard_normal((d_k, d_v))
    a, U, V = so.state_from_dense(S, vbar, R)
    S0 = so.reconstruct(a, U, V, vbar)
    steps = _steps(rule, rng, 3 * W + 3, d_k, d_v, vbar)
    a1, U1, V1, o1, _ = sc.scheduled_run(rule, a, U, V, vbar, steps, R, W, D)
    Sd, od = so.dense_run(rule, S0, steps)
    assert np.allclose(np.array(o1), np.array(od), atol=1e-9)
    assert np.allclose(so.reconstruct(a1, U1, V1, vbar), Sd, atol=1e-9)


def test_delay_changes_the_result_and_keeps_the_columns():
    """Below full rank a delay is a different schedule (the D steps see the
    uncompressed state); the column count follows columns_before_step."""
    rng = np.random.default_rng(3)
    d_k, d_v, R, W, D = 10, 8, 2, 5, 2
    vbar = rng.standard_normal(d_v)
    a, U, V = so.state_from_dense(rng.standard_normal((d_k, d_v)), vbar, R)
    steps = _steps("gdn", rng, 4 * W, d_k, d_v, vbar)
    _, _, _, o0, _ = sc.scheduled_run("gdn", a, U, V, vbar, steps, R, W, 0)
    _, _, _, oD, ev = sc.scheduled_run("gdn", a, U, V, vbar, steps, R, W, D)
    o0, oD = np.array(o0), np.array(oD)
    assert np.allclose(o0[:W], oD[:W])                  # identical until the first snapshot
    assert not np.allclose(o0[W:W + D], oD[W:W + D])   # then the delay shows
    assert [e[:2] for e in ev[:2]] == [(W, "snapshot"), (W + D, "merge")]
    for A in range(1, 4 * W):
        _, Ua, _, _, _ = sc.scheduled_run("gdn", a, U, V, vbar, steps[:A], R, W, D)
        assert Ua.shape[1] == sc.columns_before_step(A, R, W, D), A
        assert R + (A if A < W + D else D) <= Ua.shape[1] <= R + W + D
