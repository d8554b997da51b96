"""The 16-bit form (kept factors in fp16 or bf16, see include/seed.h) on the
GPU against the oracle (oracle/seed_rounding.py).

Reading under test (SEED figures and tables, Table 4 and Table 9: factors
rounded to nearest or stochastically at every compression): the R columns a
compression writes are rounded once and kept in 16 bits; appended columns
stay fp32 until the next compression.

  * seed_round_factors: bit-exact against the oracle's rounding of the same
    fp32 values, both roundings, both formats, with ties, the fp16
    subnormal range, overflow and zeros, and the generator's counter at
    high unit indices.
  * seed_decode_step_h16: W steps from a 16-bit state (no compression) --
    read-outs to 1e-4 and states to 1e-5 (relative, per unit) against the
    oracle's Lemma 2 steps on the exact widened values; appended columns are
    fp32, the 16-bit columns are never written.
  * seed_compress_h16: on the same fp32/16-bit inputs as the oracle's
    rounded compression -- every stored element is the oracle's pattern, an
    adjacent one (the fp32 result and the fp64 result may straddle a
    rounding boundary), or within the rounding bound plus 1e-5 of its
    column's norm (elements far below their column's scale, where the fp32
    error spans several spacings); at least 97% of the patterns equal; the
    rounded content within the rounding bound plus the fp32 compression
    tolerance; gam reset to 1.
  * a decode run with compressions against the oracle's own independent
    run: both are the same exact run plus their own roundings, so states
    and read-outs must agree to 4 u (u the format's relative rounding bound:
    2^-p to nearest, 2^(1-p) stochastic, p = 11 fp16, 8 bf16).
Units whose content has a near-tie at rank R, or near-equal leading
singular values (their factors are not unique), are left out of the
element-wise checks only.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TIE_GAP, TOL_READOUT, TOL_STATE_COMPRESS, TOL_STATE_STEP, f64, rel_err,
                      requires_gpu, state_rel_err, true_factors16)
from oracle import seed_rounding as rd
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

FMTS = {"bf16": (torch.bfloat16, rd.BF16, 8), "fp16": (torch.float16, rd.FP16, 11)}
# fp32 error allowed on a compressed factor element beyond its rounding,
# relative to its column's norm (the factors of a unique truncation)
TOL_FACTOR = 1e-5
SEED64 = 0x0123456789ABCDEF


def _bits(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _ordinal(bits):
    """Signed position of a pattern on the format's number line (+0 = -0 = 0)."""
    b = bits.astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def _u_store(fmt, mode):
    p = FMTS[fmt][2]
    return 2.0 ** -p if mode == "nearest" else 2.0 ** (1 - p)


# ---------------------------------------------------------------------------
# seed_round_factors: bit-exact
# ---------------------------------------------------------------------------

def _probe_tensor(shape, fmt, gen):
    """fp32 values that exercise the rounding: log-uniform magnitudes, exact
    ties of the format, zeros, the fp16 subnormal range and overflow."""
    n = int(np.prod(shape))
    mag = torch.exp2(torch.empty(n).uniform_(-30.0, 17.0, generator=gen))
    x = mag * torch.where(torch.rand(n, generator=gen) < 0.5, -1.0, 1.0)
    kind = torch.randint(0, 8, (n,), generator=gen)
    if fmt == "fp16":
        b = torch.randint(1, 0x7BFF, (n,), generator=gen, dtype=torch.int32).to(torch.int16)
        lo = b.view(torch.float16).double()
        hi = (b + 1).view(torch.float16).double()
        ties = ((lo + hi) / 2).float()
    else:
        b = torch.randint(0, 0x7F7F, (n,), generator=gen, dtype=torch.int32)
        ties = ((b << 16) | 0x8000).view(torch.float32)
    x = torch.where(kind == 1, ties, x)
    x = torch.where(kind == 2, -ties, x)
    x = torch.where(kind == 3, torch.zeros_like(x), x)
    x = torch.where(kind == 4, x * 2.0 ** -20, x)            # deep into the fp16 subnormals
    x = torch.where(kind == 5, torch.randn(n, generator=gen) * 0.1, x)
    return x.reshape(shape).contiguous()


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("mode", ["nearest", "stochastic"])
@pytest.mark.parametrize("dims,R", [((128, 128), 16), ((128, 64), 32), ((64, 64), 5)])
def test_round_factors_bit_exact(fmt, mode, dims, R):
    d_k, d_v = dims
    tdt, ofmt, _ = FMTS[fmt]
    gen = torch.Generator().manual_seed(11 + R + d_v)
    B, H = 3, 5
    U = _probe_tensor((B, H, R, d_k), fmt, gen)
    V = _probe_tensor((B, H, R, d_v), fmt, gen)
    Uk = torch.empty(B, H, R, d_k, device="cuda", dtype=tdt)
    Vk = torch.empty(B, H, R, d_v, device="cuda", dtype=tdt)
    binding.seed_round_factors(U.cuda(), V.cuda(), Uk, Vk, mode, SEED64, 7)
    torch.cuda.synchronize()
    gU = _bits(Uk).reshape(B * H, R, d_k)
    gV = _bits(Vk).reshape(B * H, R, d_v)
    Un = U.numpy().reshape(B * H, R, d_k)
    Vn = V.numpy().reshape(B * H, R, d_v)
    for u in range(B * H):
        oU, oV = rd.round_factors(Un[u].T, Vn[u].T, ofmt, mode, SEED64, 7, unit=u)
        assert np.array_equal(gU[u], oU.T), (u, np.argwhere(gU[u] != oU.T)[:4])
        assert np.array_equal(gV[u], oV.T), (u, np.argwhere(gV[u] != oV.T)[:4])


def test_round_factors_counter_at_high_units():
    """The unit index enters the generator's counter: units far apart (and
    the last of 16384) draw the oracle's words."""
    B, H, R, d_k, d_v = 512, 32, 16, 128, 128
    gen = torch.Generator().manual_seed(5)
    U = torch.randn(B, H, R, d_k, generator=gen) * 0.1
    V = torch.randn(B, H, R, d_v, generator=gen)
    Uk = torch.empty(B, H, R, d_k, device="cuda", dtype=torch.float16)
    Vk = torch.empty(B, H, R, d_v, device="cuda", dtype=torch.float16)
    binding.seed_round_factors(U.cuda(), V.cuda(), Uk, Vk, "stochastic", 99, 123456)
    torch.cuda.synchronize()
    Un, Vn = U.numpy().reshape(-1, R, d_k), V.numpy().reshape(-1, R, d_v)
    gU, gV = _bits(Uk).reshape(-1, R, d_k), _bits(Vk).reshape(-1, R, d_v)
    for u in (0, 1, 4095, 9001, B * H - 1):
        oU, oV = rd.round_factors(Un[u].T, Vn[u].T, rd.FP16, "stochastic", 99, 123456, unit=u)
        assert np.array_equal(gU[u], oU.T) and np.array_equal(gV[u], oV.T), u


# ---------------------------------------------------------------------------
# a 16-bit state built from seeded inputs
# ---------------------------------------------------------------------------

B, H = 4, 8


def _h16_state(rule, d_k, d_v, R, W, w0, fmt, seed, rounding="nearest"):
    """A state w0 steps after a compression: orthonormal-ish kept U, kept V
    with decaying column scales (both stored as 16-bit inputs), w0 fp32
    appended columns, gam in (0.5, 1).  Everything here is input data."""
    tdt = FMTS[fmt][0]
    gen = torch.Generator().manual_seed(seed)
    vbar = torch.randn(H, d_v, generator=gen)
    st = binding.ShallowState16(rule, B, H, d_k, d_v, R, W, vbar.cuda(), store=tdt,
                                rounding=rounding, seed=SEED64)
    U0 = torch.linalg.qr(torch.randn(B, H, d_k, R, generator=gen))[0].transpose(-1, -2)
    scale = torch.exp(-0.15 * torch.arange(R, dtype=torch.float32))
    V0 = torch.randn(B, H, R, d_v, generator=gen) * scale[:, None] * 3.0
    st.a.copy_(torch.randn(B, H, d_k, generator=gen).cuda())
    st.Uk.copy_(U0.to(tdt).cuda())
    st.Vk.copy_(V0.to(tdt).cuda())
    kw = torch.randn(B, H, w0, d_k, generator=gen)
    st.Uw[:, :, :w0] = (kw / kw.norm(dim=-1, keepdim=True) * 1.3).cuda()
    st.Vw[:, :, :w0] = (torch.randn(B, H, w0, d_v, generator=gen) * 0.3).cuda()
    gshape = (B, H, d_k) if rule == "kda" else (B, H)
    st.gam.copy_((0.5 + 0.5 * torch.rand(gshape, generator=gen)).cuda())
    st.r = R + w0
    return st, vbar


def _state_np(st):
    """(a, U at true scale [n, d_k, r], V [n, d_v, r]) of every unit, fp64."""
    U, V = true_factors16(st)
    return (f64(st.a).reshape(-1, st.d_k), f64(U).reshape(B * H, st.r, st.d_k).transpose(0, 2, 1),
            f64(V).reshape(B * H, st.r, st.d_v).transpose(0, 2, 1))


def _oracle_state(st):
    """The same state from the raw inputs, exactly, in fp64 (gam applied in
    fp64, not through the device)."""
    w = st.r - st.R
    Uf = np.concatenate([f64(st.Uk.float()), f64(st.Uw)[:, :, :w]], axis=2)
    Vf = np.concatenate([f64(st.Vk.float()), f64(st.Vw)[:, :, :w]], axis=2)
    gam = f64(st.gam)
    gs = gam if st.rule == "kda" else gam[..., None]
    Uf = Uf * gs[:, :, None, :]
    return (f64(st.a).reshape(-1, st.d_k), Uf.reshape(B * H, st.r, st.d_k).transpose(0, 2, 1),
            Vf.reshape(B * H, st.r, st.d_v).transpose(0, 2, 1))


def _inputs_np(x):
    return {k: (None if t is None else f64(t).reshape((B * H,) + tuple(t.shape[2:])))
            for k, t in x.items()}


# ---------------------------------------------------------------------------
# seed_decode_step_h16
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("rule,dims,R,W,in_dtype", [
    ("gdn", (128, 128), 16, 32, torch.bfloat16), ("kda", (128, 128), 16, 64, torch.bfloat16),
    ("mamba2", (128, 64), 16, 32, torch.bfloat16), ("gdn", (64, 64), 16, 20, torch.float32),
    ("kda", (128, 64), 32, 64, torch.float32)])
def test_step_h16_matches_oracle(fmt, rule, dims, R, W, in_dtype):
    d_k, d_v = dims
    st, vbar = _h16_state(rule, d_k, d_v, R, W, 3, fmt, 31 + R + W)
    a, U, V = _oracle_state(st)
    vb = np.broadcast_to(f64(vbar)[None], (B, H, d_v)).reshape(-1, d_v)
    Uk0, Vk0 = st.Uk.clone(), st.Vk.clone()
    o = torch.empty(B, H, d_v, device="cuda")
    for t in range(W - 3):
        x = wl.make_step(rule, B, H, d_k, d_v, st.vbar, 310 + R, t, 0, in_dtype, "cuda")
        st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        a, U, V, o_ref = oracle.seed_step(rule, a, U, V, vb, **_inputs_np(x))
        assert rel_err(f64(o).reshape(-1, d_v), o_ref, -1).max() < TOL_READOUT, t
        ga, gU, gV = _state_np(st)
        assert state_rel_err(ga, gU, gV, a, U, V, vb).max() < TOL_STATE_STEP, t
    assert st.r == R + W
    assert torch.equal(st.Uk, Uk0) and torch.equal(st.Vk, Vk0)
    with pytest.raises(binding.SeedError, match="SEED_E_FULL"):
        st.step(x["q"], x["k"], x["v"], x["g"], x["beta"], o)


# ---------------------------------------------------------------------------
# seed_compress_h16
# ---------------------------------------------------------------------------

def _unique_factors(U, V, R, gap=1e-3):
    """True where the rank-R factors are unique up to column signs: a clear
    gap at rank R and between every pair of the leading R + 1 singular
    values (relative to the largest)."""
    s = np.linalg.svd(U @ np.swapaxes(V, -1, -2), compute_uv=False)
    top = s[..., : R + 1]
    d = -np.diff(top, axis=-1) / np.maximum(s[..., :1], 1e-300)
    return np.all(d > gap, axis=-1)


@pytest.mark.parametrize("fmt", ["bf16", "fp16"])
@pytest.mark.parametrize("mode", ["nearest", "stochastic"])
@pytest.mark.parametrize("rule,dims,R,W", [
    ("gdn", (128, 128), 16, 32), ("kda", (128, 128), 16, 64), ("mamba2", (128, 64), 16, 32),
    ("gdn", (64, 64), 16, 24), ("kda", (128, 64), 32, 64)])
def test_compress_h16_matches_oracle(fmt, mode, rule, dims, R, W):
    d_k, d_v = dims
    tdt, ofmt, _ = FMTS[fmt]
    st, vbar = _h16_state(rule, d_k, d_v, R, W, W, fmt, 51 + R + W, rounding=mode)
    st.epoch = 5
    a0, U, V = _oracle_state(st)
    Uw0, Vw0 = st.Uw.clone(), st.Vw.clone()
    st.compress()
    torch.cuda.synchronize()
    assert st.r == R and st.epoch == 6
    assert torch.equal(st.gam, torch.ones_like(st.gam))
    assert torch.equal(st.Uw, Uw0) and torch.equal(st.Vw, Vw0)
    vb = np.broadcast_to(f64(vbar)[None], (B, H, d_v)).reshape(-1, d_v)
    gU = _bits(st.Uk).reshape(B * H, R, d_k)
    gV = _bits(st.Vk).reshape(B * H, R, d_v)
    u_st = _u_store(fmt, mode)
    tie = oracle.trunc_svd(U @ np.swapaxes(V, -1, -2), R)[2]
    gap_ok = (tie[:, R - 1] - tie[:, R]) / tie[:, 0] > TIE_GAP
    uniq = _unique_factors(U, V, R) & gap_ok
    assert uniq.sum() >= B * H // 2, "too few units with unique factors for the element checks"
    equal = total = 0
    worst = 0.0
    for u in range(B * H):
        oU, oV, L, F = rd.compress_rounded(U[u], V[u], R, ofmt, mode, SEED64, 5, unit=u)
        xU, xV = rd.widen(gU[u].T, ofmt), rd.widen(gV[u].T, ofmt)
        # content: within the rounding bound of the truncation plus fp32 error
        if gap_ok[u]:
            M = L @ F.T
            err = np.linalg.norm(xU @ xV.T - M)
            bound = (2 * u_st + u_st ** 2) * np.linalg.norm(np.abs(L) @ np.abs(F).T)
            assert err <= bound + TOL_STATE_COMPRESS * np.linalg.norm(M), u
            S_g = oracle.reconstruct(a0[u], xU, xV, vb[u])
            S_o = oracle.reconstruct(a0[u], L, F, vb[u])
            assert rel_err(S_g, S_o, (-2, -1)) < 2 * u_st + TOL_STATE_COMPRESS, u
        if not uniq[u]:
            continue
        # element-wise: the oracle's pattern or an adjacent one, column signs aligned
        sgn = np.where(np.sum(xU * L, axis=0) < 0, -1, 1)
        gUa = np.where(sgn[None, :] < 0, gU[u].T ^ np.uint16(0x8000), gU[u].T)
        gVa = np.where(sgn[None, :] < 0, gV[u].T ^ np.uint16(0x8000), gV[u].T)
        for g_, o_, X in ((gUa, oU, L), (gVa, oV, F)):
            d = np.abs(_ordinal(g_) - _ordinal(o_))
            equal += int(np.count_nonzero(d == 0))
            total += d.size
            # beyond adjacent patterns only where the fp32 compression error
            # (absolute, on the scale of the column) exceeds the spacing
            x32 = X.astype(np.float32).astype(np.float64)
            sp = rd._grid(np.abs(x32), ofmt)[1]
            excess = np.abs(rd.widen(g_, ofmt) - x32) - (0.5 if mode == "nearest" else 1.0) * sp
            col = np.linalg.norm(X, axis=0)[None, :]
            worst = max(worst, float(np.max(excess / col)))
            bad = (d > 1) & (excess > TOL_FACTOR * col)
            assert not bad.any(), (u, np.argwhere(bad)[:4], float(np.max(excess / col)))
    print(f"compress_h16 {rule} {dims} {fmt} {mode}: equal patterns {equal / total:.5f}, "
          f"largest excess over the rounding bound {worst:.2e} of the column norm")
    assert equal >= 0.97 * total, equal / total


# ---------------------------------------------------------------------------
# a decode run with compressions, against the oracle's own run
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("fmt,mode", [("fp16", "nearest"), ("bf16", "nearest"),
                                      ("fp16", "stochastic"), ("bf16", "stochastic")])
@pytest.mark.parametrize("rule,dims,R,W", [("gdn", (128, 128), 16, 32),
                                           ("kda", (128, 128), 16, 64),
                                           ("mamba2", (128, 64), 16, 32)])
def test_h16_run_matches_oracle_run(fmt, mode, rule, dims, R, W):
    d_k, d_v = dims
    tdt, ofmt, _ = FMTS[fmt]
    seed = 700 + R + W
    vbar = wl.make_vbar(H, d_v, seed, 0, "cuda")
    vb = np.broadcast_to(f64(vbar)[None], (B, H, d_v)).reshape(-1, d_v)
    # dense prefill (inputs only: a seeded prefilled state, built on the CPU)
    S = np.zeros((B * H, d_k, d_v))
    for t in range(-64, 0):
        x = wl.make_step(rule, B, H, d_k, d_v, vbar.cpu(), seed, t, 0, torch.bfloat16, "cpu")
        S, _ = oracle.dense_step(rule, S, **_inputs_np(x))
    S_dev = torch.tensor(S.reshape(B, H, d_k, d_v), dtype=torch.float32, device="cuda")
    S32 = f64(S_dev).reshape(B * H, d_k, d_v)
    st = binding.ShallowState16(rule, B, H, d_k, d_v, R, W, vbar, store=tdt, rounding=mode,
                                seed=SEED64)
    st.from_dense(S_dev)
    # the oracle's own conversion and rounding (epoch 0), then its own run
    a, L, F = oracle.state_from_dense(S32, vb, R)
    Uo = np.empty_like(L)
    Vo = np.empty_like(F)
    for u in range(B * H):
        bU, bV = rd.round_factors(L[u].astype(np.float32), F[u].astype(np.float32), ofmt, mode,
                                  SEED64, 0, unit=u)
        Uo[u], Vo[u] = rd.widen(bU, ofmt), rd.widen(bV, ofmt)
    U, V = Uo, Vo
    epoch = 1
    tol = 4 * _u_store(fmt, mode)
    ok = np.ones(B * H, bool)
    o = torch.empty(B, H, d_v, device="cuda")
    for t in range(2 * W + 5):
        x = wl.make_step(rule, B, H, d_k, d_v, vbar, seed, t, 0, torch.bfloat16, "cuda")
        compressed = st.step_and_maybe_compress(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        a, U, V, o_ref = oracle.seed_step(rule, a, U, V, vb, **_inputs_np(x))
        if U.shape[-1] >= R + W:
            s = np.linalg.svd(U @ np.swapaxes(V, -1, -2), compute_uv=False)
            ok &= (s[:, R - 1] - s[:, R]) / s[:, 0] > TIE_GAP
            Un, Vn = np.empty(U.shape[:-1] + (R,)), np.empty(V.shape[:-1] + (R,))
            for u in range(B * H):
                bU, bV, _, _ = rd.compress_rounded(U[u], V[u], R, ofmt, mode, SEED64, epoch, u)
                Un[u], Vn[u] = rd.widen(bU, ofmt), rd.widen(bV, ofmt)
            U, V = Un, Vn
            epoch += 1
            assert compressed
        assert rel_err(f64(o).reshape(-1, d_v), o_ref, -1)[ok].max() < tol, t
        ga, gU, gV = _state_np(st)
        assert state_rel_err(ga, gU, gV, a, U, V, vb)[ok].max() < tol, t
    assert st.epoch == epoch and ok.sum() >= B * H // 2


# ---------------------------------------------------------------------------
# the bound step call (state checked once) against the checked call
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("form", ["in_place", "lazy", "fp16", "bf16"])
def test_bound_step_equals_step(form):
    rule, d_k, d_v, R, W = "kda", 128, 128, 16, 32
    states = []
    for _ in range(2):
        if form in ("fp16", "bf16"):
            st, vbar = _h16_state(rule, d_k, d_v, R, W, 2, form, 77)
        else:
            gen = torch.Generator().manual_seed(77)
            vbar = torch.randn(H, d_v, generator=gen)
            st = binding.ShallowState(rule, B, H, d_k, d_v, R, W, vbar.cuda(),
                                      lazy=form == "lazy")
            st.a.copy_(torch.randn(B, H, d_k, generator=gen).cuda())
            st.U[:, :, :R] = (torch.randn(B, H, R, d_k, generator=gen) * 0.1).cuda()
            st.V[:, :, :R] = torch.randn(B, H, R, d_v, generator=gen).cuda()
            st.r = R
        states.append(st)
    o1 = torch.empty(B, H, d_v, device="cuda")
    o2 = torch.empty(B, H, d_v, device="cuda")
    f = states[1].bind_step(o2)
    for t in range(W - 2):
        x = wl.make_step(rule, B, H, d_k, d_v, states[0].vbar, 5, t, 0, torch.bfloat16, "cuda")
        states[0].step(x["q"], x["k"], x["v"], x["g"], x["beta"], o1)
        f(x["q"], x["k"], x["v"], x["g"], x["beta"], states[1].r)
        states[1].r += 1
        assert torch.equal(o1, o2), t
    for name in (("Uk", "Vk", "Uw", "Vw", "gam") if form in ("fp16", "bf16") else ("U", "V")):
        assert torch.equal(getattr(states[0], name), getattr(states[1], name)), name
    assert torch.equal(states[0].a, states[1].a)
    # inputs of the wrong shape are refused before any launch; a full state
    # is refused by the library
    with pytest.raises(ValueError, match="shape"):
        f(x["q"][:, :1], x["k"], x["v"], x["g"], x["beta"], states[1].r)
    with pytest.raises(binding.SeedError, match="SEED_E_FULL"):
        f(x["q"], x["k"], x["v"], x["g"], x["beta"], R + W)


# ---------------------------------------------------------------------------
# the 16-bit form at the benchmark's launch sizes, sampled units
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("num", [2, 3, 5])
def test_h16_workload_launch_size(num):
    """Workloads 2, 3 and 5 (one layer's launch: 1024, 8192 and 8192 heads)
    in the fp16 form, as bench.py's variant runs them: GPU prefill and
    conversion of every head, then two windows with compressions.  The
    oracle prefills, converts, rounds and compresses sampled heads on its
    own from the same inputs; read-outs and states agree to 4 u (fp16 to
    nearest), plus the prefill's fp32 rounding."""
    w = wl.WORKLOADS[num]
    dev = "cuda"
    units = w.batch * w.heads
    rng = np.random.default_rng(num)
    idx = np.unique(np.concatenate([[0, units - 1], rng.integers(0, units, 4)]))
    vbar = wl.make_vbar(w.heads, w.d_v, w.seed, 0, dev)
    vb = f64(vbar)[idx % w.heads]
    S = torch.zeros(w.batch, w.heads, w.d_k, w.d_v, device=dev)
    o = torch.empty(w.batch, w.heads, w.d_v, device=dev)
    S_ref = np.zeros((len(idx), w.d_k, w.d_v))

    def sample(x):
        return {k: (None if v is None else f64(v.reshape((units,) + tuple(v.shape[2:]))[idx]))
                for k, v in x.items()}

    for t in range(-w.prefill, 0):
        x = wl.workload_step(w, vbar, t, 0, dev)
        binding.dense_decode_step(w.rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        S_ref, _ = oracle.dense_step(w.rule, S_ref, **sample(x))
    st = binding.ShallowState16(w.rule, w.batch, w.heads, w.d_k, w.d_v, w.R, w.W, vbar,
                                store=torch.float16, rounding="nearest", seed=SEED64)
    st.from_dense(S)
    # the oracle's own conversion, rounded (epoch 0), per sampled unit
    a, L, F = oracle.state_from_dense(S_ref, vb, w.R)
    U = np.empty_like(L)
    V = np.empty_like(F)
    for i, u in enumerate(idx):
        bU, bV = rd.round_factors(L[i].astype(np.float32), F[i].astype(np.float32), rd.FP16,
                                  "nearest", SEED64, 0, unit=int(u))
        U[i], V[i] = rd.widen(bU, rd.FP16), rd.widen(bV, rd.FP16)
    s0 = np.linalg.svd(S_ref - a[:, :, None] * vb[:, None, :], compute_uv=False)
    ok = (s0[:, w.R - 1] - s0[:, w.R]) / s0[:, 0] > TIE_GAP
    tol = 4 * _u_store("fp16", "nearest") + TOL_READOUT
    epoch = 1
    worst = 0.0
    for t in range(2 * w.W + 3):
        x = wl.workload_step(w, vbar, t, 0, dev)
        st.step_and_maybe_compress(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        a, U, V, o_ref = oracle.seed_step(w.rule, a, U, V, vb, **sample(x))
        if U.shape[-1] >= w.R + w.W:
            s = np.linalg.svd(U @ np.swapaxes(V, -1, -2), compute_uv=False)
            ok &= (s[:, w.R - 1] - s[:, w.R]) / s[:, 0] > TIE_GAP
            Un, Vn = np.empty(U.shape[:-1] + (w.R,)), np.empty(V.shape[:-1] + (w.R,))
            for i, u in enumerate(idx):
                bU, bV, _, _ = rd.compress_rounded(U[i], V[i], w.R, rd.FP16, "nearest", SEED64,
                                                   epoch, int(u))
                Un[i], Vn[i] = rd.widen(bU, rd.FP16), rd.widen(bV, rd.FP16)
            U, V = Un, Vn
            epoch += 1
        e = rel_err(f64(o.reshape(units, w.d_v)[idx]), o_ref, -1)[ok]
        worst = max(worst, float(e.max()) if e.size else 0.0)
        assert e.size == 0 or e.max() < tol, (t, e)
    ga = f64(st.a.reshape(units, w.d_k)[idx])
    Ut, Vt = true_factors16(st, torch.as_tensor(idx, device="cuda"))
    gU = f64(Ut).transpose(0, 2, 1)
    gV = f64(Vt).transpose(0, 2, 1)
    assert state_rel_err(ga, gU, gV, a, U, V, vb)[ok].max() < tol
    assert ok.sum() >= len(idx) - 1
    print(f"workload {num} fp16: worst read-out error {worst:.2e} (bar {tol:.2e})")
