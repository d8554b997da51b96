"""Pins of the oracle's dense recurrences (definition mode) to closed forms.

Nothing here re-types the oracle's formulas: every expected value is either
worked out by hand on a 2x2 head or is a property the recurrence must have
(exact retrieval of the delta rule, orthogonal writes, pure decay).
"""
import numpy as np
import pytest

from oracle import GDN, KDA, MAMBA2, dense_run, dense_step

S0 = np.array([[1.0, 2.0], [3.0, 4.0]])
K = np.array([1.0, 0.0])
V = np.array([5.0, 6.0])


def test_gdn_hand_example():
    # (I - 0.5 k k^T) S0 = [[0.5, 1], [3, 4]];  * g=0.5 -> [[0.25, 0.5], [1.5, 2]]
    # + beta k v^T = [[2.5, 3], [0, 0]]  ->  S' = [[2.75, 3.5], [1.5, 2]]
    S1, o = dense_step(GDN, S0, q=[1.0, 1.0], k=K, v=V, g=0.5, beta=0.5)
    np.testing.assert_allclose(S1, [[2.75, 3.5], [1.5, 2.0]], rtol=0, atol=1e-15)
    # o = S'^T q with q = (1, 1): column sums
    np.testing.assert_allclose(o, [4.25, 5.5], rtol=0, atol=1e-15)


def test_kda_hand_example_rows_are_decayed():
    # Diag(g) S0 scales ROWS (key channels): [[0.5, 1], [0.75, 1]]
    # (I - 0.5 k k^T)(...) = [[0.25, 0.5], [0.75, 1]];  + [[2.5, 3], [0, 0]]
    S1, o = dense_step(KDA, S0, q=[0.0, 1.0], k=K, v=V, g=np.array([0.5, 0.25]), beta=0.5)
    np.testing.assert_allclose(S1, [[2.75, 3.5], [0.75, 1.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o, [0.75, 1.0], rtol=0, atol=1e-15)


def test_mamba2_hand_example():
    # S' = 0.5 S0 + k v^T = [[5.5, 7], [1.5, 2]]
    S1, o = dense_step(MAMBA2, S0, q=[1.0, 0.0], k=K, v=V, g=0.5)
    np.testing.assert_allclose(S1, [[5.5, 7.0], [1.5, 2.0]], rtol=0, atol=1e-15)
    np.testing.assert_allclose(o, [5.5, 7.0], rtol=0, atol=1e-15)


@pytest.mark.parametrize("rule", [GDN, KDA])
def test_delta_rule_exact_retrieval(rule):
    """With g = 1, beta = 1 and |k| = 1 the delta rule stores v under k:
    k^T S' = v^T, whatever S was (non-square head to catch transposes)."""
    rng = np.random.default_rng(1)
    d_k, d_v = 7, 5
    S = rng.standard_normal((d_k, d_v))
    k = rng.standard_normal(d_k)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(d_v)
    g = 1.0 if rule == GDN else np.ones(d_k)
    S1, o = dense_step(rule, S, q=k, k=k, v=v, g=g, beta=1.0)
    np.testing.assert_allclose(k @ S1, v, atol=1e-13)
    np.testing.assert_allclose(o, v, atol=1e-13)      # read-out after the update


def test_gdn_partial_write_along_key():
    """Along the unit key, GDN keeps (1 - beta) of the decayed old value and
    adds beta of the new one: k^T S' = g (1 - beta) k^T S + beta v^T."""
    rng = np.random.default_rng(2)
    S = rng.standard_normal((6, 4))
    k = rng.standard_normal(6)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(4)
    g, beta = 0.83, 0.37
    S1, _ = dense_step(GDN, S, q=k, k=k, v=v, g=g, beta=beta)
    np.testing.assert_allclose(k @ S1, g * (1 - beta) * (k @ S) + beta * v, atol=1e-13)
    # orthogonal to k the state only decays
    P = np.eye(6) - np.outer(k, k)
    np.testing.assert_allclose(P @ S1, g * (P @ S), atol=1e-13)


@pytest.mark.parametrize("rule", [GDN, KDA])
def test_orthogonal_keys_closed_form(rule):
    """Writing distinct basis keys e_t into S = 0: each row t holds
    beta_t v_t decayed by the later steps' g (no delta interference)."""
    rng = np.random.default_rng(3)
    d_k, d_v, T = 5, 3, 5
    vs = rng.standard_normal((T, d_v))
    betas = rng.uniform(0.1, 1.0, T)
    gs = rng.uniform(0.5, 1.0, (T, d_k)) if rule == KDA else rng.uniform(0.5, 1.0, T)
    steps = [{"q": np.eye(d_k)[t], "k": np.eye(d_k)[t], "v": vs[t], "g": gs[t],
              "beta": betas[t]} for t in range(T)]
    S, _ = dense_run(rule, np.zeros((d_k, d_v)), steps)
    for t in range(T):
        later = gs[t + 1:, t] if rule == KDA else gs[t + 1:]
        np.testing.assert_allclose(S[t], np.prod(later) * betas[t] * vs[t], atol=1e-14)


def test_mamba2_no_decay_is_sum_of_outer_products():
    rng = np.random.default_rng(4)
    d_k, d_v, T = 6, 3, 9
    S0 = rng.standard_normal((d_k, d_v))
    ks = rng.standard_normal((T, d_k))
    vs = rng.standard_normal((T, d_v))
    steps = [{"q": ks[t], "k": ks[t], "v": vs[t], "g": 1.0} for t in range(T)]
    S, _ = dense_run(MAMBA2, S0, steps)
    np.testing.assert_allclose(S, S0 + ks.T @ vs, atol=1e-12)


@pytest.mark.parametrize("rule", [GDN, KDA])
def test_no_write_no_decay_is_static(rule):
    rng = np.random.default_rng(5)
    S0 = rng.standard_normal((4, 6))
    g = 1.0 if rule == GDN else np.ones(4)
    S1, o = dense_step(rule, S0, q=rng.standard_normal(4), k=rng.standard_normal(4),
                       v=rng.standard_normal(6), g=g, beta=0.0)
    np.testing.assert_array_equal(S1, S0)


def test_kda_pure_decay_scales_key_rows():
    rng = np.random.default_rng(6)
    S0 = rng.standard_normal((4, 6))
    g = np.array([0.1, 0.2, 0.3, 0.4])
    S1, _ = dense_step(KDA, S0, q=np.ones(4), k=rng.standard_normal(4),
                       v=rng.standard_normal(6), g=g, beta=0.0)
    np.testing.assert_allclose(S1, S0 * g[:, None], atol=1e-15)


def test_readout_picks_rows_and_batches():
    """o = S'^T q: a basis query reads one key row; leading batch dims are
    independent heads."""
    rng = np.random.default_rng(7)
    B = 3
    S = rng.standard_normal((B, 4, 5))
    k = rng.standard_normal((B, 4))
    v = rng.standard_normal((B, 5))
    g = rng.uniform(0.5, 1, B)
    beta = rng.uniform(0, 1, B)
    q = np.zeros((B, 4))
    q[:, 2] = 1.0
    S1, o = dense_step(GDN, S, q, k, v, g, beta)
    np.testing.assert_allclose(o, S1[:, 2, :], atol=1e-15)
    for b in range(B):
        Sb, ob = dense_step(GDN, S[b], q[b], k[b], v[b], g[b], beta[b])
        np.testing.assert_allclose(S1[b], Sb, atol=1e-15)
