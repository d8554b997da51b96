"""The lazily decayed form (U = Diag(gam) U~, see include/seed.h) against the
in-place form on the GPU and against the oracle.

Both forms start from the same state and take the same inputs through a
window of W steps and a compression.  Every read-out of the lazy form must
match the in-place form's to 1e-5 and the oracle's to 1e-4 (relative, per
unit); the reconstructed states must agree to 1e-5 between compressions
and 1e-4 after one; after the compression gam is exactly 1 and U~ is U."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TOL_READOUT, TOL_STATE_COMPRESS, TOL_STATE_STEP, f64, inputs_np, make_state,
                      rel_err, requires_gpu, state_np, state_rel_err, true_U)
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

B, H = 4, 8


def _true_state(st, r):
    a = f64(st.a).reshape(-1, st.d_k)
    U = f64(true_U(st)).reshape(-1, st.cap, st.d_k)[:, :r].transpose(0, 2, 1)
    V = f64(st.V).reshape(-1, st.cap, st.d_v)[:, :r].transpose(0, 2, 1)
    return a, U, V


@pytest.mark.parametrize("rule,dims,R,W", [("gdn", (128, 128), 16, 32), ("kda", (128, 128), 16, 64),
                                           ("mamba2", (128, 64), 16, 32), ("gdn", (64, 64), 8, 24)])
def test_lazy_matches_in_place_and_oracle(rule, dims, R, W):
    d_k, d_v = dims
    gen = torch.Generator(device="cuda").manual_seed(95)
    vbar = torch.randn(H, d_v, device="cuda", generator=gen)
    eager = make_state(rule, B, H, d_k, d_v, R, W, vbar)
    lazy = make_state(rule, B, H, d_k, d_v, R, W, vbar)
    lazy.lazy = True
    lazy.gam = torch.ones((B, H, d_k) if rule == "kda" else (B, H), device="cuda")
    a0 = torch.randn(B, H, d_k, device="cuda", generator=gen)
    U0 = torch.linalg.qr(torch.randn(B, H, d_k, R, device="cuda", generator=gen))[0]
    V0 = torch.randn(B, H, R, d_v, device="cuda", generator=gen)
    for st in (eager, lazy):
        st.a.copy_(a0)
        st.U[:, :, :R] = U0.transpose(-1, -2)
        st.V[:, :, :R] = V0
        st.r = R
    a, U, V, vb = state_np(eager)
    o_e = torch.empty(B, H, d_v, device="cuda")
    o_l = torch.empty(B, H, d_v, device="cuda")
    for t in range(W):
        x = wl.make_step(rule, B, H, d_k, d_v, vbar, 96, t, 0, torch.bfloat16, "cuda")
        eager.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o_e)
        lazy.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o_l)
        a, U, V, o_ref = oracle.seed_step(rule, a, U, V, vb, **inputs_np(x))
        ol = f64(o_l).reshape(-1, d_v)
        assert rel_err(ol, f64(o_e).reshape(-1, d_v), -1).max() < TOL_STATE_STEP, t
        assert rel_err(ol, o_ref, -1).max() < TOL_READOUT, t
        la, lU, lV = _true_state(lazy, lazy.r)
        assert state_rel_err(la, lU, lV, a, U, V, vb).max() < TOL_STATE_STEP, t
    gap_ok = np.ones(B * H, bool)
    eager.compress()
    lazy.compress()
    torch.cuda.synchronize()
    assert torch.equal(lazy.gam, torch.ones_like(lazy.gam))
    Uc, Vc = oracle.compress(U, V, R)
    la, lU, lV = _true_state(lazy, R)
    ea, eU, eV = _true_state(eager, R)
    assert state_rel_err(la, lU, lV, ea, eU, eV, vb)[gap_ok].max() < TOL_STATE_COMPRESS
    assert state_rel_err(la, lU, lV, a, Uc, Vc, vb)[gap_ok].max() < TOL_STATE_COMPRESS
    # after the compression the stored columns are at true scale
    assert torch.equal(true_U(lazy)[:, :, :R], lazy.U[:, :, :R].to("cpu", torch.float64))
