"""bench.py's host side without a GPU: the one-GPU rule and the algorithmic
byte account the roofline divides by."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from sink_rank_recurrent_amd import workloads as wl  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr or "single MI355X" in r.stderr


def _mean(w, form):
    rs = range(w.R, w.R + w.W)          # columns held before each step of a window
    return sum(bench.step_bytes_per_unit(w, r, form) for r in rs) / w.W


def test_step_bytes_per_head_step_workload2():
    """Workload 2 (GDN 128 x 128, bf16 q/k/v, R = 16, W = 32, 64 requests):
    the per-head-step bytes of each form, mean r = 31.5."""
    w = wl.WORKLOADS[2]
    assert _mean(w, "in_place") == pytest.approx(51728.0)
    assert _mean(w, "lazy") == pytest.approx(35608.0)
    assert _mean(w, "h16") == pytest.approx(27416.0)
    # the dense baseline reads and writes the whole state
    assert bench.dense_bytes_per_unit(w) == 8 * 128 * 128 + 2 * (2 * 128 + 128) + 4 + 4 + 4 * 128


def test_byte_account_terms():
    """Each term of the account, at one r: factors read (and U written in
    place), the appended columns, a, the inputs, the gates, vbar's share."""
    w = wl.WORKLOADS[3]            # Mamba-2 128 x 64, no beta, 128 requests
    r = 20
    d_k, d_v = w.d_k, w.d_v
    read = 4 * d_k + 4 * (d_k + d_v) * r + 2 * (2 * d_k + d_v) + 4 + 4 * d_v / w.batch
    write_in_place = 4 * d_k + 4 * d_k * (r + 1) + 4 * d_v + 4 * d_v
    assert bench.step_bytes_per_unit(w, r, "in_place") == pytest.approx(read + write_in_place)
    lazy = read + 4 + 4 * d_k + 4 * d_k + 4 * d_v + 4 * d_v + 4
    assert bench.step_bytes_per_unit(w, r, "lazy") == pytest.approx(lazy)
    h16 = lazy - 2 * (d_k + d_v) * w.R
    assert bench.step_bytes_per_unit(w, r, "h16") == pytest.approx(h16)
