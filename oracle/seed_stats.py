"""CPU oracle for the state statistics (numpy, float64).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests use it.  It shares no code with the HIP
library.

The quantities the SEED figures and tables (thelatestinai.com) measure on a
head's recurrent state S (d_k x d_v) and its direction vbar:
  * the sink a vbar^T, a = S vbar/|vbar|^2, and its share of the state's
    energy |a vbar^T|_F^2 / |S|_F^2 (Fig. 3 (b), (g));
  * the content C = S - a vbar^T (Fig. 3 (c); Lemma 1) and its energy;
  * the singular spectra of S and C (Fig. 3 (e); Fig. 13 (a)) and the top
    direction's share sigma_1(S)^2 / |S|_F^2 (Fig. 13 (b));
  * |cos| between the state's top output direction v* -- the leading right
    singular vector of S, in value space -- and vbar (Fig. 3 (h), Fig. 13 (c));
  * the smallest rank holding 90 % and 99 % of the content's energy
    (Fig. 13 (d)) and the share of the content's energy beyond rank R
    (Fig. 12 (f)).
Reading: energy is the squared Frobenius norm, shared out over squared
singular values; "rank holding p" is the smallest k with
sum_{i<=k} sigma_i(C)^2 >= p |C|_F^2 (0 for a zero content).

Pins: tests/test_oracle_stats.py (planted spectra, a pure sink, a state
with a known top direction, brute force over ranks).
"""
from __future__ import annotations

import numpy as np

from .seed_oracle import sink_extract

# the record of one head (order of the fields the GPU writes)
FIELDS = ("e_state", "e_sink", "e_content", "sink_share", "top_share", "abs_cos_vstar_vbar",
          "rank90", "rank99", "beyond_R_share")


def rank_holding(s2, p):
    """Smallest k with sum of the k largest s2 >= p * total (0 if total is 0)."""
    s2 = np.sort(np.asarray(s2, np.float64))[::-1]
    tot = s2.sum()
    if tot <= 0:
        return 0
    c = np.cumsum(s2)
    return int(np.argmax(c >= p * tot) + 1)


def state_stats(S, vbar, R):
    """Statistics of one head (S [d_k, d_v], vbar [d_v]) as a dict, plus the
    squared singular values of S and of C (descending)."""
    S = np.asarray(S, np.float64)
    vbar = np.asarray(vbar, np.float64)
    a, C = sink_extract(S, vbar)
    e_state = float(np.sum(S * S))
    e_sink = float(np.sum(a * a) * np.sum(vbar * vbar))
    e_content = float(np.sum(C * C))
    _, sS, Vt = np.linalg.svd(S)
    sC = np.linalg.svd(C, compute_uv=False)
    s2S, s2C = sS ** 2, sC ** 2
    vstar = Vt[0]
    cos = abs(float(vstar @ vbar)) / float(np.linalg.norm(vbar))
    out = {
        "e_state": e_state, "e_sink": e_sink, "e_content": e_content,
        "sink_share": e_sink / e_state if e_state > 0 else 0.0,
        "top_share": float(s2S[0]) / e_state if e_state > 0 else 0.0,
        "abs_cos_vstar_vbar": cos,
        "rank90": rank_holding(s2C, 0.90), "rank99": rank_holding(s2C, 0.99),
        "beyond_R_share": float(np.sum(s2C[R:])) / e_content if e_content > 0 else 0.0,
    }
    return out, s2S, s2C
