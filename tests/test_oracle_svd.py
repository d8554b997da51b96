"""Pins of the oracle's sink extraction and rank-R truncation.

Expected values come from constructions whose answer is known without an
SVD (prescribed spectra, a 2x2 matrix solved by hand, a brute-force search
over rank-1 approximations), never from re-calling the routine the oracle
uses.
"""
import numpy as np
import pytest

from oracle import compress, reconstruct, sink_extract, state_from_dense, trunc_svd


def _orthonormal(rng, m, n):
    Q, Rr = np.linalg.qr(rng.standard_normal((m, n)))
    return Q * np.sign(np.diag(Rr))


def test_sink_extract_recovers_planted_split():
    """S = a vbar^T + C with C vbar = 0 -> extraction returns exactly (a, C).
    vbar is deliberately not unit-norm."""
    rng = np.random.default_rng(10)
    d_k, d_v = 9, 6
    vbar = 3.7 * rng.standard_normal(d_v)
    a = rng.standard_normal(d_k)
    C = rng.standard_normal((d_k, d_v))
    C -= np.outer(C @ vbar, vbar) / (vbar @ vbar)
    a2, C2 = sink_extract(np.outer(a, vbar) + C, vbar)
    np.testing.assert_allclose(a2, a, atol=1e-13)
    np.testing.assert_allclose(C2, C, atol=1e-13)
    np.testing.assert_allclose(C2 @ vbar, 0, atol=1e-12)


def test_sink_of_rank_one_along_vbar():
    vbar = np.array([0.0, 2.0, 0.0])
    S = np.outer([1.0, -2.0], vbar)
    a, C = sink_extract(S, vbar)
    np.testing.assert_allclose(a, [1.0, -2.0])
    np.testing.assert_allclose(C, 0)


@pytest.mark.parametrize("m,n,R", [(12, 8, 3), (8, 12, 5), (16, 16, 16), (6, 4, 7)])
def test_trunc_prescribed_spectrum(m, n, R):
    rng = np.random.default_rng(11 + m + n + R)
    p = min(m, n)
    P = _orthonormal(rng, m, p)
    Q = _orthonormal(rng, n, p)
    s = np.sort(rng.uniform(0.5, 4.0, p))[::-1] * (1.0 + np.arange(p)[::-1] * 0.2)
    s = np.sort(s)[::-1]
    C = P @ np.diag(s) @ Q.T
    L, F, sv = trunc_svd(C, R)
    kept = min(R, p)
    np.testing.assert_allclose(sv, s, rtol=1e-12)
    expect = P[:, :kept] @ np.diag(s[:kept]) @ Q[:, :kept].T
    np.testing.assert_allclose(L @ F.T, expect, atol=1e-12)
    # Eckart-Young error identity
    err2 = np.sum((C - L @ F.T) ** 2)
    np.testing.assert_allclose(err2, np.sum(s[kept:] ** 2), atol=1e-11)
    # U orthonormal, V carries the singular values, missing rank is zero
    np.testing.assert_allclose(L[:, :kept].T @ L[:, :kept], np.eye(kept), atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(F[:, :kept], axis=0), s[:kept], rtol=1e-12)
    assert L.shape == (m, R) and F.shape == (n, R)
    np.testing.assert_array_equal(L[:, kept:], 0)
    np.testing.assert_array_equal(F[:, kept:], 0)


def test_trunc_two_by_two_by_hand():
    # C = [[3, 0], [4, 5]]: C^T C = [[25, 20], [20, 25]], eigenvalues 45 and 5,
    # so s = (3 sqrt5, sqrt5); right vector (1, 1)/sqrt2, left (1, 3)/sqrt10;
    # the rank-1 truncation is s1 u1 v1^T = 1.5 [[1, 1], [3, 3]].
    C = np.array([[3.0, 0.0], [4.0, 5.0]])
    L, F, s = trunc_svd(C, 1)
    np.testing.assert_allclose(s, [3 * np.sqrt(5), np.sqrt(5)], rtol=1e-14)
    np.testing.assert_allclose(L @ F.T, [[1.5, 1.5], [4.5, 4.5]], atol=1e-14)


def test_trunc_rank1_brute_force():
    """Search every unit left direction u (fine grid on the circle): the best
    rank-1 approximation with left factor u is u (u^T C), with error
    |C|^2 - |u^T C|^2.  The truncation must reach the grid's minimum."""
    rng = np.random.default_rng(12)
    C = rng.standard_normal((2, 5))
    th = np.linspace(0.0, np.pi, 200001)
    Us = np.stack([np.cos(th), np.sin(th)])
    err2 = np.sum(C * C) - np.sum((Us.T @ C) ** 2, axis=1)
    L, F, _ = trunc_svd(C, 1)
    got = np.sum((C - L @ F.T) ** 2)
    assert got <= err2.min() + 1e-12
    assert got >= err2.min() - 1e-8


def test_state_from_dense_keeps_sink_and_truncates_content():
    rng = np.random.default_rng(13)
    d_k, d_v, R = 10, 7, 3
    vbar = rng.standard_normal(d_v)
    S = rng.standard_normal((d_k, d_v))
    a, U, V = state_from_dense(S, vbar, R)
    np.testing.assert_allclose(a, S @ vbar / (vbar @ vbar), atol=1e-13)
    np.testing.assert_allclose(V.T @ vbar, 0, atol=1e-12)    # content orthogonal to vbar
    # the truncated content is the best rank-R fit: residual equals tail energy
    C = S - np.outer(a, vbar)
    s = np.linalg.svd(C, compute_uv=False)
    res = np.sum((S - reconstruct(a, U, V, vbar)) ** 2)
    np.testing.assert_allclose(res, np.sum(s[R:] ** 2), rtol=1e-10)


def test_compress_matches_prescribed_product():
    rng = np.random.default_rng(14)
    d_k, d_v, n, R = 16, 12, 9, 4
    # U V^T with a known spectrum: U = P diag(s), V = Q (n = rank)
    P = _orthonormal(rng, d_k, n)
    Q = _orthonormal(rng, d_v, n)
    s = np.linspace(5.0, 1.0, n)
    M = rng.standard_normal((n, n))
    Mi = np.linalg.inv(M)
    U = P @ np.diag(s) @ M          # the factors need not be orthogonal
    V = Q @ Mi.T                    # U V^T = P diag(s) Q^T
    U2, V2 = compress(U, V, R)
    np.testing.assert_allclose(U2 @ V2.T, P[:, :R] @ np.diag(s[:R]) @ Q[:, :R].T, atol=1e-11)
    np.testing.assert_allclose(U2.T @ U2, np.eye(R), atol=1e-12)
