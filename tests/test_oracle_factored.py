"""Pins of the oracle's factored mode (Lemma 2 and compression) against its
definition mode and against what the pages fix: exactness between
compressions, the sink's own recurrence, invariants, special cases and the
open-loop error bound of Corollary 4.
"""
import numpy as np
import pytest

from oracle import (GDN, KDA, MAMBA2, RULES, compress, define_run, dense_run, dense_step,
                    factored_run, reconstruct, seed_step, sink_extract, state_from_dense)


def _inputs(rng, rule, T, d_k, d_v, vbar, lead=(), g_lo=0.9, g_hi=0.999):
    steps = []
    for _ in range(T):
        k = rng.standard_normal(lead + (d_k,))
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q = rng.standard_normal(lead + (d_k,))
        q /= np.linalg.norm(q, axis=-1, keepdims=True)
        v = vbar + 0.3 * rng.standard_normal(lead + (d_v,))
        if rule == KDA:
            g = rng.uniform(g_lo, g_hi, lead + (d_k,))
        else:
            g = rng.uniform(g_lo, g_hi, lead)
        beta = None if rule == MAMBA2 else rng.uniform(0, 1, lead)
        steps.append({"q": q, "k": k, "v": v, "g": g, "beta": beta})
    return steps


def _prefill(rng, rule, d_k, d_v, vbar, T=40, lead=()):
    S, _ = dense_run(rule, np.zeros(lead + (d_k, d_v)), _inputs(rng, rule, T, d_k, d_v, vbar, lead))
    return S


@pytest.mark.parametrize("rule", RULES)
def test_lemma2_step_equals_dense_step(rule):
    """Any factored state, one step: a+ vbar^T + U+ V+^T equals the dense
    recurrence applied to a vbar^T + U V^T, and the read-outs agree."""
    rng = np.random.default_rng(20)
    lead, d_k, d_v, r = (3, 2), 9, 7, 5
    vbar = rng.standard_normal(lead + (d_v,))
    a = rng.standard_normal(lead + (d_k,))
    U = rng.standard_normal(lead + (d_k, r))
    V = rng.standard_normal(lead + (d_v, r))
    (inp,) = _inputs(rng, rule, 1, d_k, d_v, vbar, lead)
    a1, U1, V1, o1 = seed_step(rule, a, U, V, vbar, **inp)
    S1, o2 = dense_step(rule, reconstruct(a, U, V, vbar), **inp)
    assert U1.shape[-1] == r + 1 and V1.shape[-1] == r + 1
    np.testing.assert_allclose(reconstruct(a1, U1, V1, vbar), S1, atol=1e-12)
    np.testing.assert_allclose(o1, o2, atol=1e-12)


@pytest.mark.parametrize("rule", RULES)
def test_sink_follows_its_own_recurrence(rule):
    """Lemma 1: starting from a converted state, the factored a stays equal to
    the sink coefficient S vbar/|vbar|^2 of the dense trajectory, step after
    step, and the content stays orthogonal to vbar (V^T vbar = 0)."""
    rng = np.random.default_rng(21)
    d_k, d_v, R = 12, 8, 3
    vbar = rng.standard_normal(d_v)
    S = _prefill(rng, rule, d_k, d_v, vbar)
    a, U, V = state_from_dense(S, vbar, R)
    S = reconstruct(a, U, V, vbar)
    for inp in _inputs(rng, rule, 20, d_k, d_v, vbar):
        a, U, V, _ = seed_step(rule, a, U, V, vbar, **inp)
        S, _ = dense_step(rule, S, **inp)
        a_dense, _ = sink_extract(S, vbar)
        np.testing.assert_allclose(a, a_dense, atol=1e-11)
        np.testing.assert_allclose(V.T @ vbar, 0, atol=1e-11)


@pytest.mark.parametrize("rule", RULES)
def test_factored_run_equals_definition_run(rule):
    """Factored mode (Lemma 2 + compression of U V^T) and definition mode
    (dense recurrence + truncation of the extracted content) are the same
    computation; compressions included."""
    rng = np.random.default_rng(22)
    lead, d_k, d_v, R, W, T = (2,), 10, 8, 3, 4, 17
    vbar = rng.standard_normal(lead + (d_v,))
    S0 = _prefill(rng, rule, d_k, d_v, vbar, lead=lead)
    steps = _inputs(rng, rule, T, d_k, d_v, vbar, lead)
    S_def, o_def, errs = define_run(rule, S0, vbar, steps, R, W)
    a, U, V = state_from_dense(S0, vbar, R)
    a, U, V, o_fac = factored_run(rule, a, U, V, vbar, steps, R, W)
    assert U.shape[-1] == R + T % W
    np.testing.assert_allclose(reconstruct(a, U, V, vbar), S_def, atol=1e-10)
    for x, y in zip(o_fac, o_def):
        np.testing.assert_allclose(x, y, atol=1e-10)
    assert len(errs) == T // W and all(np.all(e > 0) for e in errs)


@pytest.mark.parametrize("rule", RULES)
def test_rank_at_least_content_rank_is_lossless(rule):
    """With R >= min(d_k, d_v) the truncation is exact, so the whole factored
    trajectory equals the uncompressed dense recurrence."""
    rng = np.random.default_rng(23)
    d_k, d_v, R, W, T = 6, 4, 4, 3, 13
    vbar = rng.standard_normal(d_v)
    S0 = _prefill(rng, rule, d_k, d_v, vbar)
    steps = _inputs(rng, rule, T, d_k, d_v, vbar)
    S_ref, o_ref = dense_run(rule, S0, steps)
    a, U, V = state_from_dense(S0, vbar, R)
    a, U, V, o = factored_run(rule, a, U, V, vbar, steps, R, W)
    np.testing.assert_allclose(reconstruct(a, U, V, vbar), S_ref, atol=1e-11)
    np.testing.assert_allclose(np.array(o), np.array(o_ref), atol=1e-11)


def test_static_state_without_write_or_decay():
    rng = np.random.default_rng(24)
    d_k, d_v, R = 8, 6, 3
    vbar = rng.standard_normal(d_v)
    a, U, V = state_from_dense(rng.standard_normal((d_k, d_v)), vbar, R)
    S0 = reconstruct(a, U, V, vbar)
    for rule in (GDN, KDA):
        steps = _inputs(rng, rule, 5, d_k, d_v, vbar)
        for s in steps:
            s["beta"] = 0.0
            s["g"] = np.ones_like(s["g"])
        a2, U2, V2, _ = factored_run(rule, a, U, V, vbar, steps, R, 100)
        np.testing.assert_allclose(reconstruct(a2, U2, V2, vbar), S0, atol=1e-13)
        np.testing.assert_array_equal(V2[:, R:], 0)        # appended columns are zero


def test_mamba2_value_along_vbar_appends_zero_columns():
    rng = np.random.default_rng(25)
    d_k, d_v, R = 8, 5, 2
    vbar = rng.standard_normal(d_v)
    a, U, V = state_from_dense(rng.standard_normal((d_k, d_v)), vbar, R)
    k = rng.standard_normal(d_k)
    a2, U2, V2, _ = seed_step(MAMBA2, a, U, V, vbar, q=k, k=k, v=2.5 * vbar, g=0.7)
    np.testing.assert_allclose(V2[:, -1], 0, atol=1e-15)
    np.testing.assert_allclose(a2, 0.7 * a + 2.5 * k, atol=1e-14)


@pytest.mark.parametrize("rule", RULES)
def test_corollary4_open_loop_bound(rule):
    """SEED summary (picx.dev), "Open-Loop Error Bound (Corollary 4)": with
    inputs fixed in advance, |S~_t - S_t|_F <= eps_max / (1 - g_max^W),
    where eps_max is the largest single compression error and g_max < 1 the
    largest decay.  Decays are kept well below 1 so the bound is not slack."""
    rng = np.random.default_rng(26)
    d_k, d_v, R, W, T = 12, 10, 2, 3, 30
    vbar = rng.standard_normal(d_v)
    S0 = _prefill(rng, rule, d_k, d_v, vbar)
    steps = _inputs(rng, rule, T, d_k, d_v, vbar, g_lo=0.6, g_hi=0.85)
    a, U, V = state_from_dense(S0, vbar, R)
    S_exact = reconstruct(a, U, V, vbar)       # same start for both runs
    g_max = max(float(np.max(s["g"])) for s in steps)
    S_tilde = S_exact.copy()
    eps_max = 0.0
    worst_ratio = 0.0
    for t, inp in enumerate(steps, start=1):
        S_exact, _ = dense_step(rule, S_exact, **inp)
        S_tilde, _ = dense_step(rule, S_tilde, **inp)
        if t % W == 0:
            a_t, C = sink_extract(S_tilde, vbar)
            Uc, Vc = compress(C, np.eye(d_v), R)
            new = np.outer(a_t, vbar) + Uc @ Vc.T
            eps_max = max(eps_max, np.linalg.norm(new - S_tilde))
            S_tilde = new
        err = np.linalg.norm(S_tilde - S_exact)
        bound = eps_max / (1 - g_max ** W)
        assert err <= bound * (1 + 1e-9) + 1e-12
        if eps_max > 0:
            worst_ratio = max(worst_ratio, err / bound)
    assert eps_max > 1e-3          # compression did cost something
    assert worst_ratio > 0.2       # and the bound is not vacuous here


@pytest.mark.parametrize("rule", RULES)
def test_lemma2_with_vanishing_gates(rule):
    """Gates from 5e-3 to 2e-2 for a whole window (their product falls to
    1e-50 and below): the factored run still reproduces the dense recurrence
    step by step (Lemma 2 holds for any gate), so the oracle is the right
    reference for the lazily decayed forms in that regime."""
    rng = np.random.default_rng(41)
    d_k, d_v, R, W = 12, 10, 3, 24
    vbar = rng.standard_normal(d_v)
    S0 = _prefill(rng, rule, d_k, d_v, vbar)
    a, U, V = state_from_dense(S0, vbar, R)
    S = reconstruct(a, U, V, vbar)
    for inp in _inputs(rng, rule, W, d_k, d_v, vbar, g_lo=5e-3, g_hi=2e-2):
        a, U, V, o1 = seed_step(rule, a, U, V, vbar, **inp)
        S, o2 = dense_step(rule, S, **inp)
        np.testing.assert_allclose(reconstruct(a, U, V, vbar), S, rtol=0, atol=1e-12 * np.abs(S).max())
        np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12 * np.abs(o2).max())


@pytest.mark.parametrize("rule", RULES)
def test_zero_gate_forgets_everything(rule):
    """g = 0 erases the state: Gated DeltaNet and KDA keep exactly
    beta k v^T, Mamba-2 exactly k v^T, whatever came before (the dense
    recurrences with g = 0), and the factored step gives the same."""
    rng = np.random.default_rng(42)
    d_k, d_v, R = 9, 7, 3
    vbar = rng.standard_normal(d_v)
    a, U, V = state_from_dense(_prefill(rng, rule, d_k, d_v, vbar), vbar, R)
    (inp,) = _inputs(rng, rule, 1, d_k, d_v, vbar)
    inp["g"] = np.zeros_like(inp["g"])
    a1, U1, V1, o = seed_step(rule, a, U, V, vbar, **inp)
    b = 1.0 if rule == MAMBA2 else inp["beta"]
    expect = b * np.outer(inp["k"], inp["v"])
    np.testing.assert_allclose(reconstruct(a1, U1, V1, vbar), expect, atol=1e-14)
    np.testing.assert_allclose(o, expect.T @ inp["q"], atol=1e-14)
