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
SRC = os.path.join(ROOT, "oracle", "seed_oracle.py")
PIN_FILES = ["tests/test_oracle_dense.py", "tests/test_oracle_svd.py",
             "tests/test_oracle_factored.py", "tests/test_oracle_bytes.py"]

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

RUNNER = r"""
import sys
sys.path.insert(0, sys.argv[1])
import oracle  # the mutated copy
assert oracle.__file__.startswith(sys.argv[1]), oracle.__file__
import pytest
sys.exit(pytest.main(sys.argv[2:] + ["-x", "-q", "-p", "no:cacheprovider"]))
"""


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    pkg = tmp_path / "oracle"
    pkg.mkdir()
    (pkg / "seed_oracle.py").write_text(src.replace(old, new))
    (pkg / "__init__.py").write_text(open(os.path.join(ROOT, "oracle", "__init__.py")).read())
    r = subprocess.run([sys.executable, "-c", RUNNER, str(tmp_path)] + PIN_FILES,
                       cwd=ROOT, capture_output=True, text=True, timeout=300)
    assert r.returncode != 0, f"mutation {name} survived the pins:\n{r.stdout[-2000:]}"
