"""The oracle's pins must catch plausible mistakes.

Each case copies the oracle, plants one mistake in the copy (a dropped term,
a flipped sign, a wrong operand or index), and runs the oracle pin tests
against the copy in a subprocess: at least one pin must fail.  The real
oracle is never modified.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")
PIN_FILES = ["tests/test_oracle_dense.py", "tests/test_oracle_svd.py",
             "tests/test_oracle_factored.py", "tests/test_oracle_bytes.py"]
ROUNDING_PINS = ["tests/test_oracle_rounding.py"]
STATS_PINS = ["tests/test_oracle_stats.py"]

MUTATIONS = {
    "lemma2_sign_of_kGa": ("(beta * (omega - kGa))", "(beta * (omega + kGa))"),
    "lemma2_undecayed_U_in_c": ("c = (np.swapaxes(GU, -1, -2) @ k", "c = (np.swapaxes(U, -1, -2) @ k"),
    "lemma2_dropped_beta_on_column": ("v_col = beta[..., None] * (eps - ", "v_col = (eps - "),
    "mamba2_value_not_split": ("        v_col = eps\n", "        v_col = v\n"),
    "readout_before_update": ("vbar * np.sum(a_new * q, axis=-1)", "vbar * np.sum(a * q, axis=-1)"),
    "kda_decay_on_wrong_side": ("(eye - b * kkT) @ (g[..., :, None] * S)", "((eye - b * kkT) @ S) * g[..., :, None]"),
    "gdn_missing_delta_term": ("((eye - b * kkT) @ S)", "(S)"),
    "sink_norm_not_squared": ("/ np.sum(vbar * vbar, axis=-1)[..., None]",
                              "/ np.sqrt(np.sum(vbar * vbar, axis=-1))[..., None]"),
    "trunc_keeps_smallest": ("L[..., :, :kept] = P[..., :, :kept]", "L[..., :, :kept] = P[..., :, -kept:]"),
    "trunc_drops_sigma": ("* s[..., None, :kept]", "* 1.0"),
    "bytes_counts_vbar": ("return b_s * (d_k + (d_k + d_v) * (R + w))",
                          "return b_s * (d_k + d_v + (d_k + d_v) * (R + w))"),
    "define_compress_every_step": ("if t % W == 0:\n            a, C = sink_extract",
                                   "if True:\n            a, C = sink_extract"),
}

# mistakes planted in the 16-bit storage oracle (seed_rounding.py)
ROUNDING_MUTATIONS = {
    "philox_no_key_bump": ("        if rnd:\n            k0 = (k0 + np.uint64(_W0)) & _MASK",
                           "        if False:\n            k0 = (k0 + np.uint64(_W0)) & _MASK"),
    "philox_swapped_products": ("p1 & _MASK,\n", "p0 & _MASK,\n"),
    "nearest_ties_away": ("up = (frac > 0.5) | ((frac == 0.5) & tie_up)", "up = frac >= 0.5"),
    "nearest_no_subnormal_binade": ("e = np.maximum(ex - 1, emin)", "e = ex - 1"),
    "stochastic_compares_ge": ("np.where(frac > u, lo + sp, lo)", "np.where(frac >= u, lo + sp, lo)"),
    "stochastic_u_from_low_bits": ("(np.asarray(words, dtype=np.uint32) >> 8)",
                                   "(np.asarray(words, dtype=np.uint32) & 0xFFFFFF)"),
    "words_v_block_not_offset": ("w[R * d_k:].reshape(R, d_v).T", "w[:R * d_v].reshape(R, d_v).T"),
    "compress_scales_a_factor": ("round_factors(L.astype(np.float32), F.astype(np.float32)",
                                    "round_factors(L.astype(np.float32) * 1.001, F.astype(np.float32)"),
}

# mistakes planted in the state-statistics oracle (seed_stats.py)
STATS_MUTATIONS = {
    "sink_energy_norm_not_squared": ("np.sum(a * a) * np.sum(vbar * vbar)",
                                     "np.sum(a * a) * np.sqrt(np.sum(vbar * vbar))"),
    "rank_holding_strict": ("np.argmax(c >= p * tot)", "np.argmax(c > p * tot)"),
    "vstar_from_last_direction": ("vstar = Vt[0]", "vstar = Vt[-1]"),
    "beyond_rank_off_by_one": ("np.sum(s2C[R:])", "np.sum(s2C[R + 1:])"),
    "top_share_of_content": ("float(s2S[0]) / e_state", "float(s2C[0]) / e_state"),
}

RUNNER = r"""
import sys
sys.path.insert(0, sys.argv[1])
import oracle  # the mutated copy
assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__
import pytest
sys.exit(pytest.main(sys.argv[2:] + ["-x", "-q", "-p", "no:cacheprovider"]))
"""


def _run_mutated(tmp_path, fname, old, new, pins):
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    for f in os.listdir(ORACLE):
        if f.endswith(".py"):
            src = open(os.path.join(ORACLE, f)).read()
            if f == fname:
                assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
                src = src.replace(old, new)
            (pkg / f).write_text(src)
    return subprocess.run([sys.executable, "-c", RUNNER, str(tmp_path)] + pins,
                          cwd=ROOT, capture_output=True, text=True, timeout=300)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    r = _run_mutated(tmp_path, "seed_oracle.py", old, new, PIN_FILES)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(ROUNDING_MUTATIONS))
def test_planted_rounding_mistake_is_caught(name, tmp_path):
    old, new = ROUNDING_MUTATIONS[name]
    r = _run_mutated(tmp_path, "seed_rounding.py", old, new, ROUNDING_PINS)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"


@pytest.mark.parametrize("name", sorted(STATS_MUTATIONS))
def test_planted_stats_mistake_is_caught(name, tmp_path):
    old, new = STATS_MUTATIONS[name]
    r = _run_mutated(tmp_path, "seed_stats.py", old, new, STATS_PINS)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
