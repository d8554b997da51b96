"""CPU oracle for per-request (staggered) compression schedules (fp64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests use it.  It shares no code with the HIP
library.

The pages compress every W steps (SEED figures and tables on
thelatestinai.com, Fig. 1 (b) caption) and serve requests that start at
different times (Fig. 8).  Reading used here for a request that has taken A
steps since its state was converted (its column count is its own):
  * after the step that brings its window to W columns (A = k W, k >= 1),
    the content [kept R columns | W window columns] is taken as a snapshot
    and its rank-R truncation computed;
  * the request keeps taking exact Lemma 2 steps on its full state, which
    appends D more columns;
  * D steps after the snapshot (A = k W + D) the snapshot's columns are
    replaced by the truncation -- decayed by the gates of those D steps, as
    every column of U is -- and the D columns appended since are kept;
  * D = 0 is compression at the snapshot itself, the aligned reading per
    request.
So a request holds R + w columns with w in [D, W + D) once it has been
compressed, and w = A before.

Pins: tests/test_oracle_schedule.py (D = 0 equals the factored run; with R at
full rank nothing is lost, so every D reproduces the dense recurrence; the
column counts).
"""
from __future__ import annotations

import numpy as np

from .seed_oracle import GDN, KDA, MAMBA2, compress, seed_step


def _decay_cols(rule, U, g):
    """G U for one step's gate: g scalar (GDN, Mamba-2) or per key channel."""
    if rule == KDA:
        return np.asarray(g)[:, None] * U
    return float(g) * U


def scheduled_run(rule, a, U, V, vbar, steps, R, W, D):
    """Run one unit from (a, U [d_k, R], V [d_v, R]) through `steps` (dicts
    of q, k, v, g, beta for this unit) under the schedule above.

    Returns (a, U, V, outs, events): the final state (true-scale U), the
    read-outs, and the events in order: (A, "snapshot", gap, tail) with
    gap = (s_R - s_{R+1}) / s_1 and tail = s_{R+1} / s_1 of the snapshot's
    content (the truncation is unique only where gap is positive; where tail
    is at the rounding level every truncation is as good), and (A, "merge")."""
    if not 0 <= D < W:
        raise ValueError("need 0 <= D < W")
    a, U, V, vbar = (np.asarray(x, np.float64) for x in (a, U, V, vbar))
    outs, events = [], []
    pend = None           # (truncated U at true scale, V, column count at the snapshot)
    for A, x in enumerate(steps, start=1):
        a, U, V, o = seed_step(rule, a, U, V, vbar, x["q"], x["k"], x["v"], x["g"], x.get("beta"))
        outs.append(o)
        if pend is not None:
            # the truncation decays with the state it will replace
            pend = (_decay_cols(rule, pend[0], x["g"]), pend[1], pend[2])
        if A % W == 0:
            L, F = compress(U, V, R)
            pend = (L, F, U.shape[-1])
            s = np.linalg.svd(U @ V.T, compute_uv=False)
            gap = (s[R - 1] - s[R]) / s[0] if s.size > R and s[0] > 0 else 1.0
            tail = s[R] / s[0] if s.size > R and s[0] > 0 else 0.0
            events.append((A, "snapshot", float(gap), float(tail)))
        if pend is not None and A % W == D:
            L, F, n0 = pend
            U = np.concatenate([L, U[:, n0:]], axis=1)
            V = np.concatenate([F, V[:, n0:]], axis=1)
            pend = None
            events.append((A, "merge"))
    return a, U, V, outs, events


def columns_before_step(A, R, W, D):
    """Columns a request holds before its step number A + 1 (A steps taken)."""
    if A < W + D:
        return R + A
    c = (A - D) // W
    return R + A - c * W
