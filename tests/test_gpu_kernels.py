"""Per-call parity of every entry point with the CPU oracle, on identical
inputs (bf16 inputs are compared through their exact fp64 values).

Sizes: 15 (request, head) units (3 x 5, a ragged count of workgroups), every
head shape the library supports, and column counts r that leave ragged
tails in the 8 column groups of the step kernel (0, 1, 7, 9, 31, 47) or sit
at the capacity limit.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import (TIE_GAP, TOL_READOUT, TOL_STATE_COMPRESS, TOL_STATE_STEP, content_gap, f64,
                      inputs_np, make_state, rel_err, requires_gpu, state_np, state_rel_err,
                      units_of)
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

RULES = ["gdn", "kda", "mamba2"]
DIMS = [(128, 128), (128, 64), (64, 64)]
DTYPES = [torch.float32, torch.bfloat16]
B, H = 3, 5


def _vbar(d_v, seed):
    return wl.make_vbar(H, d_v, seed, device="cuda")


def _random_factors(st, r, seed):
    """Fill a, U, V with state-like values: U columns unit-norm-ish and
    decayed, V columns orthogonal to vbar with spread norms."""
    gen = torch.Generator(device="cuda").manual_seed(seed)
    cap, d_k, d_v = st.cap, st.d_k, st.d_v
    st.a.copy_(torch.randn(B, H, d_k, generator=gen, device="cuda"))
    U = torch.randn(B, H, cap, d_k, generator=gen, device="cuda") / d_k ** 0.5
    U *= torch.rand(B, H, cap, 1, generator=gen, device="cuda") * 0.9 + 0.1
    V = torch.randn(B, H, cap, d_v, generator=gen, device="cuda")
    vb = st.vbar[None, :, None, :]
    V -= (V * vb).sum(-1, keepdim=True) / (vb * vb).sum(-1, keepdim=True) * vb
    V *= torch.rand(B, H, cap, 1, generator=gen, device="cuda") * 2.0
    st.U.copy_(U)
    st.V.copy_(V)
    st.r = r


@pytest.mark.parametrize("in_dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("dims", DIMS, ids=lambda d: f"{d[0]}x{d[1]}")
@pytest.mark.parametrize("rule", RULES)
def test_dense_step(rule, dims, in_dtype):
    d_k, d_v = dims
    vbar = _vbar(d_v, 11)
    gen = torch.Generator(device="cuda").manual_seed(12)
    S = torch.randn(B, H, d_k, d_v, generator=gen, device="cuda")
    o = torch.empty(B, H, d_v, device="cuda")
    S_ref = f64(units_of(S))            # the seeded input; the oracle runs on from it
    for t in range(3):
        inp = wl.make_step(rule, B, H, d_k, d_v, vbar, 13, t, 0, in_dtype, "cuda")
        S_ref, o_ref = oracle.dense_step(rule, S_ref, **inputs_np(inp))
        binding.dense_decode_step(rule, S, inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o)
        torch.cuda.synchronize()
        assert rel_err(f64(units_of(S)), S_ref, (-2, -1)).max() < TOL_STATE_STEP
        assert rel_err(f64(units_of(o)), o_ref, -1).max() < TOL_READOUT


@pytest.mark.parametrize("in_dtype", DTYPES, ids=["f32", "bf16"])
@pytest.mark.parametrize("dims", DIMS, ids=lambda d: f"{d[0]}x{d[1]}")
@pytest.mark.parametrize("rule", RULES)
def test_decode_step(rule, dims, in_dtype):
    d_k, d_v = dims
    R, W = 16, 32
    st = make_state(rule, B, H, d_k, d_v, R, W, _vbar(d_v, 21))
    o = torch.empty(B, H, d_v, device="cuda")
    for i, r in enumerate([0, 1, 7, 9, 16, 31, 47]):
        _random_factors(st, r, 100 + i)
        inp = wl.make_step(rule, B, H, d_k, d_v, st.vbar, 22, i, 0, in_dtype, "cuda")
        a0, U0, V0, vb = state_np(st)
        U_full_before = f64(st.U)
        st.step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o)
        torch.cuda.synchronize()
        a_ref, U_ref, V_ref, o_ref = oracle.seed_step(rule, a0, U0, V0, vb, **inputs_np(inp))
        a1, U1, V1, _ = state_np(st)
        assert st.r == r + 1
        # the step is exact arithmetic on the factors: compare them directly
        assert rel_err(a1, a_ref, -1).max() < TOL_STATE_STEP
        assert rel_err(U1, U_ref, (-2, -1)).max() < TOL_STATE_STEP
        assert state_rel_err(a1, U1, V1, a_ref, U_ref, V_ref, vb).max() < TOL_STATE_STEP
        assert rel_err(f64(units_of(o)), o_ref, -1).max() < TOL_READOUT
        # columns beyond the appended one are untouched
        np.testing.assert_array_equal(f64(st.U)[:, :, r + 1:], U_full_before[:, :, r + 1:])


def _oracle_precompress_states(rule, d_k, d_v, R, n, seed, units=4):
    """Realistic factors just before a compression, produced by the oracle:
    a short dense prefill, conversion, then n - R exact steps."""
    rng = np.random.default_rng(seed)
    vbar = rng.standard_normal(d_v)

    def inp():
        k = rng.standard_normal((units, d_k)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
        q = rng.standard_normal((units, d_k)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
        v = vbar + 0.3 * rng.standard_normal((units, d_v))
        if rule == "kda":
            g = rng.uniform(0.95, 0.9999, (units, d_k))
        elif rule == "gdn":
            g = rng.uniform(0.9, 0.999, units)
        else:
            g = np.exp(-np.logaddexp(0, rng.standard_normal(units)) * 0.1)
        beta = None if rule == "mamba2" else rng.uniform(0, 1, units)
        return dict(q=q, k=k, v=v, g=g, beta=beta)

    S = np.zeros((units, d_k, d_v))
    for _ in range(48):
        S, _ = oracle.dense_step(rule, S, **inp())
    a, U, V = oracle.state_from_dense(S, vbar, R)
    for _ in range(n - R):
        a, U, V, _ = oracle.seed_step(rule, a, U, V, vbar, **inp())
    return a, U, V, vbar


@pytest.mark.parametrize("rule,dims,R,W,n", [
    ("gdn", (128, 128), 16, 32, 48),
    ("gdn", (128, 128), 16, 16, 32),
    ("gdn", (128, 128), 16, 32, 33),     # compress before the ring is full, odd n
    ("kda", (128, 128), 16, 64, 80),
    ("kda", (128, 128), 32, 64, 96),     # largest capacity
    ("gdn", (128, 128), 16, 48, 64),     # one wave holding 64 columns
    ("kda", (128, 128), 16, 48, 57),     # 49 .. 64 columns, odd n
    ("gdn", (128, 128), 24, 24, 48),     # R above 16: the layout with separate late regions
    ("mamba2", (128, 64), 16, 32, 48),
    ("mamba2", (128, 64), 16, 32, 47),
    ("gdn", (64, 64), 8, 24, 32),
    ("gdn", (128, 128), 1, 8, 9),
])
def test_compress(rule, dims, R, W, n):
    d_k, d_v = dims
    units = B * H
    a, U, V, vbar_np = _oracle_precompress_states(rule, d_k, d_v, R, n, 31 + n, units)
    st = make_state(rule, B, H, d_k, d_v, R, W, torch.tensor(np.broadcast_to(vbar_np, (H, d_v)).copy(),
                                                             dtype=torch.float32))
    U32 = U.astype(np.float32)
    V32 = V.astype(np.float32)
    st.a.copy_(torch.tensor(a.reshape(B, H, d_k), dtype=torch.float32))
    st.U[:, :, :n] = torch.tensor(U32.transpose(0, 2, 1).reshape(B, H, n, d_k), device="cuda")
    st.V[:, :, :n] = torch.tensor(V32.transpose(0, 2, 1).reshape(B, H, n, d_v), device="cuda")
    st.r = n
    a_before = f64(st.a).copy()
    st.compress()
    torch.cuda.synchronize()
    assert st.r == R
    Ug, Vg = state_np(st)[1:3]
    Uc, Vc = oracle.compress(U32.astype(np.float64), V32.astype(np.float64), R)
    gap = content_gap(U32.astype(np.float64), V32.astype(np.float64), R)
    ok = gap >= TIE_GAP
    assert ok.sum() >= units - 1, f"too many near-ties: {gap}"
    prod_g = Ug @ np.swapaxes(Vg, -1, -2)
    prod_r = Uc @ np.swapaxes(Vc, -1, -2)
    S_ref = oracle.reconstruct(a.reshape(units, d_k), Uc, Vc, np.broadcast_to(vbar_np, (units, d_v)))
    err_state = np.sqrt(np.sum((prod_g - prod_r) ** 2, axis=(-2, -1))) / np.sqrt(
        np.sum(S_ref ** 2, axis=(-2, -1)))
    err_content = rel_err(prod_g, prod_r, (-2, -1))
    assert err_state[ok].max() < TOL_STATE_COMPRESS, err_state
    assert err_content[ok].max() < 1e-3, err_content
    # U' orthonormal, the sink untouched (bit for bit)
    gram = np.swapaxes(Ug, -1, -2) @ Ug
    assert np.abs(gram - np.eye(R)).max() < 1e-4
    np.testing.assert_array_equal(f64(st.a), a_before)


@pytest.mark.parametrize("dims,R", [((128, 128), 16), ((128, 64), 16), ((64, 64), 8),
                                    ((128, 128), 32), ((128, 64), 32), ((64, 64), 32),
                                    ((128, 128), 1), ((64, 64), 23)])
def test_state_from_dense(dims, R):
    d_k, d_v = dims
    gen = torch.Generator(device="cuda").manual_seed(41)
    vbar = wl.make_vbar(H, d_v, 42, device="cuda")
    # a dense state with a strong sink and a decaying content spectrum
    a_true = torch.randn(B, H, d_k, 1, generator=gen, device="cuda")
    L = torch.randn(B, H, d_k, 40, generator=gen, device="cuda")
    Rm = torch.randn(B, H, 40, d_v, generator=gen, device="cuda") * torch.logspace(
        0, -3, 40, device="cuda")[:, None]
    S = (a_true * vbar[None, :, None, :] + L @ Rm * 0.3).contiguous()
    st = make_state("gdn", B, H, d_k, d_v, R, 16, vbar)
    st.from_dense(S)
    torch.cuda.synchronize()
    assert st.r == R
    vb = np.broadcast_to(f64(vbar)[None], (B, H, d_v)).reshape(-1, d_v)
    a_r, U_r, V_r = oracle.state_from_dense(f64(units_of(S)), vb, R)
    a_g, U_g, V_g, _ = state_np(st)
    assert rel_err(a_g, a_r, -1).max() < TOL_STATE_STEP
    C = f64(units_of(S)) - a_r[..., :, None] * vb[..., None, :]
    gap = content_gap(C, np.broadcast_to(np.eye(d_v), C.shape[:-2] + (d_v, d_v)), R)
    ok = gap >= TIE_GAP
    assert ok.sum() >= B * H - 1
    err = state_rel_err(a_g, U_g, V_g, a_r, U_r, V_r, vb)
    assert err[ok].max() < TOL_STATE_COMPRESS, err
    assert np.abs(np.swapaxes(U_g, -1, -2) @ U_g - np.eye(R)).max() < 1e-4
    # the content stays orthogonal to vbar
    assert (np.abs(np.swapaxes(V_g, -1, -2) @ vb[..., :, None]).max()
            < 1e-4 * np.abs(V_g).max() * np.linalg.norm(vb, axis=-1).max())


# ---------------------------------------------------------------------------
# edge cases and degenerate inputs
# ---------------------------------------------------------------------------

def test_step_is_deterministic():
    """Two runs of the same step from the same state give identical bits
    (one workgroup owns a unit; no atomics, fixed reduction order)."""
    st = make_state("gdn", B, H, 128, 128, 16, 32, _vbar(128, 61))
    _random_factors(st, 29, 62)
    inp = wl.make_step("gdn", B, H, 128, 128, st.vbar, 63, 0, 0, torch.bfloat16, "cuda")
    saved = [t.clone() for t in (st.a, st.U, st.V)]
    outs = []
    for _ in range(2):
        st.a.copy_(saved[0]); st.U.copy_(saved[1]); st.V.copy_(saved[2]); st.r = 29
        o = torch.empty(B, H, 128, device="cuda")
        st.step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (st.a, st.U, st.V, o)])
    for x, y in zip(*outs):
        assert torch.equal(x, y)


@pytest.mark.parametrize("rule", ["gdn", "kda"])
def test_no_write_no_decay_keeps_state(rule):
    st = make_state(rule, B, H, 128, 128, 16, 32, _vbar(128, 64))
    _random_factors(st, 20, 65)
    a0, U0, V0, vb = state_np(st)
    inp = wl.make_step(rule, B, H, 128, 128, st.vbar, 66, 0, 0, torch.float32, "cuda")
    inp["beta"] = torch.zeros_like(inp["beta"])
    inp["g"] = torch.ones_like(inp["g"])
    o = torch.empty(B, H, 128, device="cuda")
    st.step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o)
    torch.cuda.synchronize()
    a1, U1, V1, _ = state_np(st)
    np.testing.assert_array_equal(a1, a0)
    np.testing.assert_array_equal(U1[..., :20], U0)
    np.testing.assert_array_equal(V1[..., 20], 0.0)        # the appended V column is zero
    assert state_rel_err(a1, U1, V1, a0, U0, V0, vb).max() == 0.0


def test_mamba2_value_along_vbar():
    st = make_state("mamba2", B, H, 128, 64, 16, 32, _vbar(64, 67))
    _random_factors(st, 17, 68)
    inp = wl.make_step("mamba2", B, H, 128, 64, st.vbar, 69, 0, 0, torch.float32, "cuda")
    inp["v"] = (2.5 * st.vbar).expand(B, H, 64).contiguous()
    a0 = f64(st.a)
    o = torch.empty(B, H, 64, device="cuda")
    st.step(inp["q"], inp["k"], inp["v"], inp["g"], None, o)
    torch.cuda.synchronize()
    newcol = f64(st.V)[:, :, 17]
    assert np.abs(newcol).max() < 1e-5 * np.abs(f64(st.vbar)).max() * 2.5
    g = f64(inp["g"])[..., None]
    np.testing.assert_allclose(f64(st.a), g * a0 + 2.5 * f64(inp["k"]), rtol=1e-5, atol=1e-6)


def test_nan_stays_in_its_unit():
    """NaN inputs are not checked: they propagate into that unit's outputs
    and nowhere else."""
    st = make_state("gdn", B, H, 128, 128, 16, 32, _vbar(128, 70))
    _random_factors(st, 12, 71)
    inp = wl.make_step("gdn", B, H, 128, 128, st.vbar, 72, 0, 0, torch.float32, "cuda")
    inp["v"][1, 2, 5] = float("nan")
    o = torch.empty(B, H, 128, device="cuda")
    st.step(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], o)
    torch.cuda.synchronize()
    on = torch.isnan(o).any(dim=-1)
    assert on[1, 2] and on.sum() == 1
    assert torch.isnan(st.a[1, 2]).any() and torch.isnan(st.a).any(dim=-1).sum() == 1


@pytest.mark.parametrize("W", [32, 64])   # one wave (n = 48), two waves (n = 80)
@pytest.mark.parametrize("case", ["dup_keys", "near_dup_keys", "zero_v_cols", "all_zero_v", "zero_u_cols"])
def test_compress_degenerate(case, W):
    d_k = d_v = 128
    R = 16
    n = R + W
    rng = np.random.default_rng(73 + W)
    units = B * H
    U = rng.standard_normal((units, d_k, n)) / np.sqrt(d_k)
    V = rng.standard_normal((units, d_v, n))
    if case == "dup_keys":
        U[:, :, 30] = 0.7 * U[:, :, 5]
        U[:, :, 41] = U[:, :, 40]
        if n > 64:
            # a column of the second wave repeats one of the first
            U[:, :, 70] = -U[:, :, 10]
    elif case == "near_dup_keys":
        # keys at angles with sines 1e-3 .. 1e-2 from earlier ones (unit by
        # unit), the rest of the column orthogonal noise of that size
        for j, i in ((30, 5), (41, 40), (47, 17)):
            sines = np.geomspace(1e-3, 1e-2, units)[rng.permutation(units)]
            base = U[:, :, i] / np.linalg.norm(U[:, :, i], axis=-1, keepdims=True)
            noise = rng.standard_normal((units, d_k))
            noise -= np.sum(noise * base, axis=-1, keepdims=True) * base
            noise /= np.linalg.norm(noise, axis=-1, keepdims=True)
            U[:, :, j] = np.sqrt(1 - sines[:, None] ** 2) * base + sines[:, None] * noise
    elif case == "zero_v_cols":
        V[:, :, 16:] = 0.0
    elif case == "all_zero_v":
        V[:] = 0.0
    else:
        U[:, :, 20:] = 0.0
    U = U.astype(np.float32).astype(np.float64)
    V = V.astype(np.float32).astype(np.float64)
    st = make_state("gdn", B, H, d_k, d_v, R, W, torch.randn(H, d_v))
    st.U[:, :, :n] = torch.tensor(U.transpose(0, 2, 1).reshape(B, H, n, d_k), dtype=torch.float32)
    st.V[:, :, :n] = torch.tensor(V.transpose(0, 2, 1).reshape(B, H, n, d_v), dtype=torch.float32)
    st.r = n
    st.compress()
    torch.cuda.synchronize()
    Ug, Vg = state_np(st)[1:3]
    assert np.isfinite(Ug).all() and np.isfinite(Vg).all()
    Uc, Vc = oracle.compress(U, V, R)
    P = Uc @ np.swapaxes(Vc, -1, -2)
    Pg = Ug @ np.swapaxes(Vg, -1, -2)
    scale = np.maximum(np.sqrt(np.sum((U @ np.swapaxes(V, -1, -2)) ** 2, axis=(-2, -1))), 1e-30)
    err = np.sqrt(np.sum((Pg - P) ** 2, axis=(-2, -1))) / scale
    ok = content_gap(U, V, R) >= TIE_GAP if case != "all_zero_v" else np.ones(units, bool)
    assert err[ok].max() < 1e-4, err


def test_from_dense_of_pure_sink():
    vbar = _vbar(128, 74)
    a_true = torch.randn(B, H, 128, 1, device="cuda")
    S = (a_true * vbar[None, :, None, :]).contiguous()
    st = make_state("gdn", B, H, 128, 128, 16, 16, vbar)
    st.from_dense(S)
    torch.cuda.synchronize()
    a, U, V, vb = state_np(st)
    np.testing.assert_allclose(a, f64(a_true)[..., 0].reshape(-1, 128), rtol=1e-5, atol=1e-6)
    prod = U @ np.swapaxes(V, -1, -2)
    assert np.abs(prod).max() < 1e-5 * np.abs(f64(S)).max()


@pytest.mark.parametrize("e", [-40, 40])
def test_far_from_unit_scale(e):
    """States scaled by 2^-40 or 2^40: the eigensolver works on H brought to
    unit range by a power of two, so neither squares below the normal range
    (read as zero by sqrt and rcp) nor squares above fp32's range break the
    conversion or the compression; both stay within the usual bar of the
    oracle on the same scaled inputs."""
    s = 2.0 ** e
    # conversion of a graded dense state
    d_k = d_v = 128
    R = 16
    gen = torch.Generator(device="cuda").manual_seed(81)
    vbar = _vbar(d_v, 82)
    a_true = torch.randn(B, H, d_k, 1, generator=gen, device="cuda")
    L = torch.randn(B, H, d_k, 40, generator=gen, device="cuda")
    Rm = torch.randn(B, H, 40, d_v, generator=gen, device="cuda") * torch.logspace(
        0, -3, 40, device="cuda")[:, None]
    S = ((a_true * vbar[None, :, None, :] + L @ Rm * 0.3) * s).contiguous()
    st = make_state("gdn", B, H, d_k, d_v, R, 16, vbar)
    st.from_dense(S)
    torch.cuda.synchronize()
    vb = np.broadcast_to(f64(vbar)[None], (B, H, d_v)).reshape(-1, d_v)
    a_r, U_r, V_r = oracle.state_from_dense(f64(units_of(S)), vb, R)
    a_g, U_g, V_g, _ = state_np(st)
    assert np.isfinite(U_g).all() and np.isfinite(V_g).all()
    C = f64(units_of(S)) - a_r[..., :, None] * vb[..., None, :]
    ok = content_gap(C, np.broadcast_to(np.eye(d_v), C.shape[:-2] + (d_v, d_v)), R) >= TIE_GAP
    assert ok.sum() >= B * H - 1
    err = state_rel_err(a_g, U_g, V_g, a_r, U_r, V_r, vb)
    assert err[ok].max() < TOL_STATE_COMPRESS, err

    # compression of factors whose content is scaled by s
    n, W = 48, 32
    a, U, V, vbar_np = _oracle_precompress_states("gdn", d_k, d_v, R, n, 83, B * H)
    U32 = (U * 2.0 ** (e // 2)).astype(np.float32)
    V32 = (V * 2.0 ** (e - e // 2)).astype(np.float32)
    st = make_state("gdn", B, H, d_k, d_v, R, W,
                    torch.tensor(np.broadcast_to(vbar_np, (H, d_v)).copy(), dtype=torch.float32))
    st.a.copy_(torch.tensor(a.reshape(B, H, d_k), dtype=torch.float32))
    st.U[:, :, :n] = torch.tensor(U32.transpose(0, 2, 1).reshape(B, H, n, d_k), device="cuda")
    st.V[:, :, :n] = torch.tensor(V32.transpose(0, 2, 1).reshape(B, H, n, d_v), device="cuda")
    st.r = n
    st.compress()
    torch.cuda.synchronize()
    Ug, Vg = state_np(st)[1:3]
    assert np.isfinite(Ug).all() and np.isfinite(Vg).all()
    U64, V64 = U32.astype(np.float64), V32.astype(np.float64)
    Uc, Vc = oracle.compress(U64, V64, R)
    ok = content_gap(U64, V64, R) >= TIE_GAP
    assert ok.sum() >= B * H - 1
    err = rel_err(Ug @ np.swapaxes(Vg, -1, -2), Uc @ np.swapaxes(Vc, -1, -2), (-2, -1))
    assert err[ok].max() < 1e-3, err


def test_stream_copy_is_exact():
    """The bandwidth probe copies every byte, also a ragged size (not a whole
    number of passes of its grid), and touches nothing beyond."""
    n = (1 << 22) + 4 * 37                      # floats: 16 MiB plus 37 vectors
    src = torch.randn(n, device="cuda")
    dst = torch.full((n + 64,), 7.0, device="cuda")
    binding.stream_copy(src, dst[:n])
    torch.cuda.synchronize()
    assert torch.equal(dst[:n], src)
    assert torch.all(dst[n:] == 7.0)
