"""CPU oracle for SEED's decode-time shallow recurrent state (fp64, numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

It is written to be checked by eye against the SEED pages, not to be fast:
every function follows one definition or one step of the method, in the
pages' notation, in float64.  Leading batch dimensions are allowed
everywhere (they are independent (request, head) units); vbar broadcasts
against them.

Notation (SEED summary on picx.dev, "SEED Architecture" and "Exact Update
(Lemma 2)"):
  S  (d_k x d_v)  recurrent state of one head
  vbar (d_v)      fixed per-head direction, shared by requests
  a  (d_k)        sink coefficient;  the sink is a vbar^T
  U  (d_k x r), V (d_v x r)  content factors;  S = a vbar^T + U V^T
  q, k (d_k), v (d_v)  query, key and value of a step
  g               decay: a scalar per head (Gated DeltaNet, Mamba-2) or a
                  d_k-vector (Kimi Delta Attention)
  beta            write strength (Gated DeltaNet, Kimi Delta Attention)
  omega = v.vbar/|vbar|^2,  eps = v - omega vbar

Readings of points the pages leave open (each is repeated where it is used):
  * the read-out is taken from the state after the step's update;
  * the Kimi Delta Attention form of Lemma 2 substitutes Diag(g) for the
    scalar g; the Mamba-2 form is Lemma 1 with Phi = g I and no delta term;
  * compression replaces the content U V^T by its best rank-R approximation
    and never touches the sink;  U comes back with orthonormal columns and
    V carries the singular values; missing rank is padded with zero columns.

Pins: every function here is checked in tests/test_oracle_*.py against
closed forms, invariants, brute force on tiny inputs, the pages' printed
byte account (Table 2) and the pages' error bound (Corollary 4).  The
numeric values of read-outs and factors on random inputs have no printed
worked example; they are pinned through those identities only.
"""
from __future__ import annotations

import numpy as np

GDN, KDA, MAMBA2 = "gdn", "kda", "mamba2"
RULES = (GDN, KDA, MAMBA2)


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


# ---------------------------------------------------------------------------
# Definition mode: the dense recurrences
# ---------------------------------------------------------------------------

def dense_step(rule, S, q, k, v, g, beta=None):
    """One step of a head's dense recurrence, then the read-out o = S'^T q.

    The three transitions, in their literal matrix form:
      Gated DeltaNet       S' = g (I - beta k k^T) S + beta k v^T
      Kimi Delta Attention S' = (I - beta k k^T) Diag(g) S + beta k v^T
      Mamba-2              S' = g S + k v^T
    (SEED summary, picx.dev: the updates named under "Exact Update
    (Lemma 2)"; Mamba-2 uses the d_k = d_B, d_v = d_x orientation of the
    Table 17 note on thelatestinai.com.)  The read-out is of the updated
    state: the current token is visible to its own query.

    Shapes: S [..., d_k, d_v]; q, k [..., d_k]; v [..., d_v];
    g [...] (Kimi: [..., d_k]); beta [...] (unused by Mamba-2).
    Returns (S', o) with o [..., d_v].
    """
    S, q, k, v, g, beta = map(_f64, (S, q, k, v, g, beta))
    d_k = S.shape[-2]
    eye = np.eye(d_k)
    kkT = k[..., :, None] * k[..., None, :]
    kvT = k[..., :, None] * v[..., None, :]
    if rule == GDN:
        b = beta[..., None, None]
        S_new = g[..., None, None] * ((eye - b * kkT) @ S) + b * kvT
    elif rule == KDA:
        b = beta[..., None, None]
        S_new = (eye - b * kkT) @ (g[..., :, None] * S) + b * kvT
    elif rule == MAMBA2:
        S_new = g[..., None, None] * S + kvT
    else:
        raise ValueError(f"unknown rule {rule!r}")
    o = np.einsum("...kv,...k->...v", S_new, q)
    return S_new, o


def dense_run(rule, S, steps):
    """Run dense_step over a list of step-input dicts; returns (S, [o_t])."""
    outs = []
    for inp in steps:
        S, o = dense_step(rule, S, inp["q"], inp["k"], inp["v"], inp["g"], inp.get("beta"))
        outs.append(o)
    return S, outs


# ---------------------------------------------------------------------------
# Sink extraction and truncation
# ---------------------------------------------------------------------------

def sink_extract(S, vbar):
    """Split a dense state into its sink coefficient and content.

    The sink is the state's projection on the head's direction:
    a = S vbar / |vbar|^2 and C = S - a vbar^T, so that C vbar = 0
    (SEED figures and tables, thelatestinai.com, Fig. 3 (b), (c); the split
    of Lemma 1 in the picx.dev summary, "Theoretical and Practical
    Implications").  vbar is used as given, not normalised.
    Returns (a [..., d_k], C [..., d_k, d_v]).
    """
    S, vbar = _f64(S), _f64(vbar)
    a = (S @ vbar[..., :, None])[..., 0] / np.sum(vbar * vbar, axis=-1)[..., None]
    C = S - a[..., :, None] * vbar[..., None, :]
    return a, C


def trunc_svd(C, R):
    """Best rank-R approximation of C (Eckart-Young), as factors.

    With C = P diag(s) Q^T (s descending), returns L = P[:, :R] (orthonormal
    columns) and F = Q[:, :R] diag(s[:R]), so that L F^T is the rank-R
    truncation, plus the full singular values s.  If C has fewer than R
    singular values the missing columns of L and F are zero.
    C: [..., m, n] -> L [..., m, R], F [..., n, R], s [..., min(m, n)].
    """
    C = _f64(C)
    P, s, Qt = np.linalg.svd(C, full_matrices=False)
    m, n = C.shape[-2], C.shape[-1]
    kept = min(R, s.shape[-1])
    L = np.zeros(C.shape[:-2] + (m, R))
    F = np.zeros(C.shape[:-2] + (n, R))
    L[..., :, :kept] = P[..., :, :kept]
    F[..., :, :kept] = np.swapaxes(Qt[..., :kept, :], -1, -2) * s[..., None, :kept]
    return L, F, s


def state_from_dense(S, vbar, R):
    """Convert a dense state to the shallow form at rank R.

    At the end of the prefill the states are compressed to the sink plus
    rank-R factors (SEED figures and tables, thelatestinai.com, Fig. 1 (a)
    caption and Table 1): a = S vbar/|vbar|^2, then the content
    C = S - a vbar^T is truncated to rank R.  Returns (a, U, V) with
    U [..., d_k, R], V [..., d_v, R].
    """
    a, C = sink_extract(S, vbar)
    U, V, _ = trunc_svd(C, R)
    return a, U, V


def reconstruct(a, U, V, vbar):
    """S = a vbar^T + U V^T (picx.dev summary, "SEED Architecture")."""
    a, U, V, vbar = map(_f64, (a, U, V, vbar))
    return a[..., :, None] * vbar[..., None, :] + U @ np.swapaxes(V, -1, -2)


# ---------------------------------------------------------------------------
# Factored mode: Lemma 2 and compression
# ---------------------------------------------------------------------------

def value_split(v, vbar):
    """omega = v.vbar/|vbar|^2 and eps = v - omega vbar (picx.dev, Lemma 2)."""
    v, vbar = _f64(v), _f64(vbar)
    omega = np.sum(v * vbar, axis=-1) / np.sum(vbar * vbar, axis=-1)
    eps = v - omega[..., None] * vbar
    return omega, eps


def seed_step(rule, a, U, V, vbar, q, k, v, g, beta=None):
    """One exact decode step on the factored state, then the read-out.

    Lemma 2 (picx.dev summary, "Exact Update (Lemma 2)"), scalar decay g:
      a+ = g a + beta (omega - g k^T a) k
      U+ = [g U, k],   V+ = [V, beta (eps - g V U^T k)]
    Kimi Delta Attention: the same with Diag(g) in place of the scalar g,
    i.e. G a = g*a and G U = Diag(g) U:
      a+ = G a + beta (omega - k^T G a) k
      U+ = [G U, k],   V+ = [V, beta (eps - V (G U)^T k)]
    Mamba-2 (Lemma 1 with Phi = g I and a plain write k v^T):
      a+ = g a + omega k,   U+ = [g U, k],   V+ = [V, eps]
    Read-out of the updated state (SEED figures and tables, Table 1: the
    factors give the read-out): o = vbar (a+^T q) + V+ (U+^T q).

    Shapes: a [..., d_k], U [..., d_k, r], V [..., d_v, r], vbar [..., d_v].
    Returns (a+, U+ [..., d_k, r+1], V+ [..., d_v, r+1], o [..., d_v]).
    """
    a, U, V, vbar, q, k, v, g, beta = map(_f64, (a, U, V, vbar, q, k, v, g, beta))
    omega, eps = value_split(v, vbar)
    if rule in (GDN, KDA):
        if rule == GDN:
            Ga = g[..., None] * a
            GU = g[..., None, None] * U
        else:
            Ga = g * a
            GU = g[..., :, None] * U
        kGa = np.sum(k * Ga, axis=-1)
        a_new = Ga + (beta * (omega - kGa))[..., None] * k
        c = (np.swapaxes(GU, -1, -2) @ k[..., :, None])[..., 0]          # (G U)^T k
        v_col = beta[..., None] * (eps - (V @ c[..., :, None])[..., 0])
    elif rule == MAMBA2:
        a_new = g[..., None] * a + omega[..., None] * k
        GU = g[..., None, None] * U
        v_col = eps
    else:
        raise ValueError(f"unknown rule {rule!r}")
    U_new = np.concatenate([GU, k[..., :, None]], axis=-1)
    V_new = np.concatenate([V, v_col[..., :, None]], axis=-1)
    Utq = (np.swapaxes(U_new, -1, -2) @ q[..., :, None])[..., 0]
    o = vbar * np.sum(a_new * q, axis=-1)[..., None] + (V_new @ Utq[..., :, None])[..., 0]
    return a_new, U_new, V_new, o


def compress(U, V, R):
    """Compress the factors back to rank R.

    Every W steps the factors are compressed back to rank R (SEED figures
    and tables, thelatestinai.com, Fig. 1 (b) caption); this is the method's
    only approximation and the sink is left exactly as it is (sungsoo.github.io
    summary, "Decode" item of the method list).  The plainest reading of
    "compress to rank R" is the best rank-R approximation of the content
    U V^T, i.e. its truncated SVD: U' = P_R (orthonormal), V' = Q_R S_R.
    """
    U, V = _f64(U), _f64(V)
    L, F, _ = trunc_svd(U @ np.swapaxes(V, -1, -2), R)
    return L, F


# ---------------------------------------------------------------------------
# Whole decode runs
# ---------------------------------------------------------------------------

def define_run(rule, S_prefill, vbar, steps, R, W):
    """Definition mode: the dense recurrence with the content truncated.

    Start from a dense prefilled state, convert it (sink kept, content
    truncated to rank R), then run the dense recurrence; after every W-th
    step replace the content by its rank-R truncation, keeping the sink.
    Returns (S_final, [o_t], [compression error_t]) where each compression
    error is |C - trunc_R(C)|_F.
    """
    a, U, V = state_from_dense(S_prefill, vbar, R)
    S = reconstruct(a, U, V, vbar)
    outs, errs = [], []
    for t, inp in enumerate(steps, start=1):
        S, o = dense_step(rule, S, inp["q"], inp["k"], inp["v"], inp["g"], inp.get("beta"))
        outs.append(o)
        if t % W == 0:
            a, C = sink_extract(S, vbar)
            L, F, s = trunc_svd(C, R)
            errs.append(np.sqrt(np.sum(s[..., R:] ** 2, axis=-1)))
            S = a[..., :, None] * _f64(vbar)[..., None, :] + L @ np.swapaxes(F, -1, -2)
    return S, outs, errs


def factored_run(rule, a, U, V, vbar, steps, R, W):
    """Factored mode: Lemma 2 steps, compressing whenever R + W columns are held.

    Starts from (a, U, V) with r = U.shape[-1] columns; returns
    (a, U, V, [o_t]).
    """
    outs = []
    for inp in steps:
        a, U, V, o = seed_step(rule, a, U, V, vbar, inp["q"], inp["k"], inp["v"],
                               inp["g"], inp.get("beta"))
        outs.append(o)
        if U.shape[-1] >= R + W:
            U, V = compress(U, V, R)
    return a, U, V, outs


# ---------------------------------------------------------------------------
# Byte account
# ---------------------------------------------------------------------------

def dense_state_bytes(d_k, d_v, b_s=4):
    """Bytes of one dense head state: b_s d_k d_v (SEED figures and tables,
    thelatestinai.com, Table 17)."""
    return b_s * d_k * d_v


def shallow_state_bytes(d_k, d_v, R, w, b_s=4):
    """Bytes of one shallow head state w steps after a compression,
    0 <= w <= W: b_s [d_k + (d_k + d_v)(R + w)] -- the sink coefficient and
    the factors; vbar is shared by all requests and not counted (Table 17)."""
    return b_s * (d_k + (d_k + d_v) * (R + w))
