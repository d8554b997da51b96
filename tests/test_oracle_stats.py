"""Pins of the state-statistics oracle (oracle/seed_stats.py): states built
with a known sink, known spectra and a known top direction, so every
statistic has a closed form."""
import numpy as np
import pytest

from oracle import seed_stats as ss


def _orth(rng, n, k):
    return np.linalg.qr(rng.standard_normal((n, k)))[0]


def _planted(rng, d_k, d_v, vbar, a, sig):
    """S = a vbar^T + P diag(sig) Q^T with Q orthogonal to vbar."""
    k = len(sig)
    P = _orth(rng, d_k, k)
    Z = rng.standard_normal((d_v, k))
    Z -= np.outer(vbar, vbar @ Z) / (vbar @ vbar)
    Q = np.linalg.qr(Z)[0]
    return np.outer(a, vbar) + P @ np.diag(sig) @ Q.T


def test_planted_content_spectrum_and_sink():
    rng = np.random.default_rng(0)
    d_k, d_v = 32, 24
    vbar = rng.standard_normal(d_v)
    a = rng.standard_normal(d_k) * 3
    sig = np.array([4.0, 2.0, 1.0, 0.5, 0.25])
    S = _planted(rng, d_k, d_v, vbar, a, sig)
    st, s2S, s2C = ss.state_stats(S, vbar, R=2)
    e_sink = np.sum(a * a) * np.sum(vbar * vbar)
    e_cont = np.sum(sig ** 2)
    assert np.isclose(st["e_sink"], e_sink) and np.isclose(st["e_content"], e_cont)
    # the content is orthogonal to the sink in value space: energies add
    assert np.isclose(st["e_state"], e_sink + e_cont)
    assert np.isclose(st["sink_share"], e_sink / (e_sink + e_cont))
    assert np.allclose(s2C[:5], sig ** 2) and np.allclose(s2C[5:], 0, atol=1e-20)
    assert np.isclose(st["beyond_R_share"], np.sum(sig[2:] ** 2) / e_cont)
    # 16 + 4 = 20 of 21.3125: 93.8 % at rank 2, 98.5 % at 3, 99.7 % at 4
    assert st["rank90"] == 2 and st["rank99"] == 4
    assert np.isclose(np.sum(s2S), st["e_state"])


def test_pure_sink():
    rng = np.random.default_rng(1)
    vbar = rng.standard_normal(16)
    a = rng.standard_normal(20)
    st, s2S, s2C = ss.state_stats(np.outer(a, vbar), vbar, R=4)
    assert np.isclose(st["sink_share"], 1.0) and np.isclose(st["top_share"], 1.0)
    assert np.isclose(st["abs_cos_vstar_vbar"], 1.0)
    # only rounding noise is left as content
    assert st["e_content"] < 1e-24 * st["e_state"]


def test_top_direction_and_its_cosine():
    """S = sigma x y^T + small orthogonal rest: v* = y, so |cos| = |y.vbar|/|vbar|."""
    rng = np.random.default_rng(2)
    d_k, d_v = 16, 12
    x = _orth(rng, d_k, 1)[:, 0]
    Yq = _orth(rng, d_v, 3)
    y = Yq[:, 0]
    vbar = rng.standard_normal(d_v)
    P = _orth(rng, d_k, 3)
    P[:, 0] = x
    P = np.linalg.qr(P)[0]
    S = 10 * np.outer(P[:, 0], y) + 1 * np.outer(P[:, 1], Yq[:, 1]) + 0.5 * np.outer(P[:, 2], Yq[:, 2])
    st, s2S, _ = ss.state_stats(S, vbar, R=1)
    assert np.isclose(st["abs_cos_vstar_vbar"], abs(y @ vbar) / np.linalg.norm(vbar))
    assert np.isclose(st["top_share"], 100 / 101.25)
    assert np.allclose(s2S[:3], [100, 1, 0.25])


def test_rank_holding_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(50):
        s2 = rng.exponential(size=rng.integers(1, 20)) ** 3
        for p in (0.9, 0.99):
            k = ss.rank_holding(s2, p)
            srt = np.sort(s2)[::-1]
            # smallest k by brute force
            want = min(j for j in range(1, len(s2) + 1) if srt[:j].sum() >= p * s2.sum())
            assert k == want
    assert ss.rank_holding(np.zeros(5), 0.9) == 0
    # exactly at the threshold: that rank holds it (0.9 * 10 and 0.99 * 100 are exact)
    assert ss.rank_holding([9.0, 1.0], 0.9) == 1
    assert ss.rank_holding([1.0, 99.0], 0.99) == 1
