"""State statistics (seed_state_stats) on the GPU against the oracle
(oracle/seed_stats.py), on the same fp32 dense states.

Bars (fp32 against fp64 SVD).  Every energy is a sum of d_k d_v squares
taken as two nested fp32 sums of at most 128 terms (a Gram entry, then a
trace or a Rayleigh quotient), each within 128 * 2^-24 = 7.6e-6 relative,
so about 1.5e-5 in all at worst; the bars leave a factor of three:
energies to 5e-5 relative; shares to 5e-5 absolute; squared singular
values to 5e-5 of the largest; |cos(v*, vbar)| to 1e-4 where the top
direction is unique ((s_1^2 - s_2^2)/s_1^2 > 1e-3); a rank is accepted if
it holds the energy share to within 5e-5 of the total and one less does
not (the decision at the threshold is taken in fp32)."""
import numpy as np
import pytest
import torch

from gpu_util import f64, requires_gpu
from oracle import seed_oracle as so
from oracle import seed_stats as ss
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _planted(rng, n, d_k, d_v, vbar):
    """Sinks plus contents with decaying planted spectra (as input data)."""
    S = np.empty((n, d_k, d_v))
    for u in range(n):
        vb = vbar[u]
        k = min(d_k, d_v) - 1
        P = np.linalg.qr(rng.standard_normal((d_k, k)))[0]
        Z = rng.standard_normal((d_v, k))
        Z -= np.outer(vb, vb @ Z) / (vb @ vb)
        Q = np.linalg.qr(Z)[0]
        sig = np.exp(-rng.uniform(0.05, 0.4) * np.arange(k)) * rng.uniform(0.2, 2.0)
        S[u] = np.outer(rng.standard_normal(d_k) * rng.uniform(0.5, 4), vb) + P @ np.diag(sig) @ Q.T
    return S


def _prefilled(rule, B, H, d_k, d_v, vbar_t, steps, seed):
    S = np.zeros((B * H, d_k, d_v))
    for t in range(-steps, 0):
        x = wl.make_step(rule, B, H, d_k, d_v, vbar_t, seed, t, 0, torch.bfloat16, "cpu")
        xi = {k: (None if v is None else f64(v).reshape((B * H,) + tuple(v.shape[2:])))
              for k, v in x.items()}
        S, _ = so.dense_step(rule, S, **xi)
    return S


TOL = 5e-5


def _rank_ok(k, s2, p, tol=TOL):
    srt = np.sort(s2)[::-1]
    tot = srt.sum()
    c = np.concatenate([[0.0], np.cumsum(srt)])
    return c[k] >= (p - tol) * tot and c[k - 1] < (p + tol) * tot


@pytest.mark.parametrize("kind", ["planted", "gdn", "kda", "mamba2"])
@pytest.mark.parametrize("dims", [(128, 128), (128, 64), (64, 64)])
def test_stats_match_oracle(kind, dims):
    d_k, d_v = dims
    if kind == "mamba2" and dims != (128, 64):
        pytest.skip("Mamba-2 heads are 128 x 64")
    B, H, R = 3, 4, 16
    rng = np.random.default_rng(["planted", "gdn", "kda", "mamba2"].index(kind) * 1000 + d_v + d_k)
    vbar_t = torch.tensor(rng.standard_normal((H, d_v)), dtype=torch.float32)
    vbar = np.broadcast_to(vbar_t.double().numpy()[None], (B, H, d_v)).reshape(-1, d_v)
    if kind == "planted":
        S = _planted(rng, B * H, d_k, d_v, vbar)
    else:
        S = _prefilled(kind, B, H, d_k, d_v, vbar_t, 96, 31)
    S32 = torch.tensor(S.reshape(B, H, d_k, d_v), dtype=torch.float32)
    S64 = S32.double().numpy().reshape(B * H, d_k, d_v)
    nf = binding.lib().seed_stat_fields()
    rec = torch.full((B, H, nf), -1.0, device="cuda")
    spS = torch.empty(B, H, d_k, device="cuda")
    spC = torch.empty(B, H, d_k, device="cuda")
    binding.seed_state_stats(S32.cuda(), vbar_t.cuda(), R, rec, spS, spC)
    torch.cuda.synchronize()
    rec = f64(rec).reshape(B * H, nf)
    spS, spC = f64(spS).reshape(B * H, d_k), f64(spC).reshape(B * H, d_k)
    worst = 0.0
    for u in range(B * H):
        want, s2S, s2C = ss.state_stats(S64[u], vbar[u], R)
        got = dict(zip(binding.STAT_FIELDS, rec[u]))
        for f in ("e_state", "e_sink", "e_content"):
            assert abs(got[f] - want[f]) <= TOL * want["e_state"], (u, f, got[f], want[f])
        for f in ("sink_share", "top_share", "beyond_R_share"):
            assert abs(got[f] - want[f]) <= TOL, (u, f, got[f], want[f])
        m = min(d_k, d_v)
        assert np.all(np.abs(spS[u, :m] - s2S[:m]) <= TOL * s2S[0]), u
        assert np.all(np.abs(spS[u, m:]) <= TOL * s2S[0]), u
        assert np.all(np.abs(spC[u, :m] - s2C[:m]) <= TOL * s2S[0]), u
        worst = max(worst, max(abs(got[f] - want[f]) for f in ("sink_share", "top_share")))
        if (s2S[0] - s2S[1]) / s2S[0] > 1e-3:
            assert abs(got["abs_cos_vstar_vbar"] - want["abs_cos_vstar_vbar"]) <= 1e-4, u
        for f, p in (("rank90", 0.90), ("rank99", 0.99)):
            k = int(got[f])
            assert k == want[f] or _rank_ok(k, s2C, p), (u, f, k, want[f])
        assert np.all(rec[u, len(binding.STAT_FIELDS):] == 0.0)
    print(f"stats {kind} {dims}: largest share error {worst:.2e}")


def test_stats_of_a_pure_sink_and_of_zero():
    """A state that is all sink: share 1, |cos| 1, no content; a zero state:
    all zeros (nothing divides by zero)."""
    B, H, d_k, d_v = 1, 2, 128, 128
    g = torch.Generator().manual_seed(4)
    vbar = torch.randn(H, d_v, generator=g)
    a = torch.randn(H, d_k, generator=g)
    S = torch.zeros(B, H, d_k, d_v)
    S[0, 0] = torch.outer(a[0], vbar[0])
    nf = binding.lib().seed_stat_fields()
    rec = torch.full((B, H, nf), -1.0, device="cuda")
    binding.seed_state_stats(S.cuda(), vbar.cuda(), 16, rec)
    torch.cuda.synchronize()
    r0 = dict(zip(binding.STAT_FIELDS, f64(rec[0, 0])))
    assert abs(r0["sink_share"] - 1) < TOL and abs(r0["top_share"] - 1) < TOL
    assert abs(r0["abs_cos_vstar_vbar"] - 1) < 1e-4
    assert r0["e_content"] <= TOL * r0["e_state"]
    assert np.all(f64(rec[0, 1]) == 0.0)
