"""Handoff of shallow-form states (seed_pack_states / seed_unpack_states)
on the GPU against the oracle's byte layout (oracle/seed_handoff.py).

Byte work, so the bar is bit-exact: the packed buffer equals the oracle's
packing of the same state, including the parts an out-of-range index must
leave untouched; unpacking writes exactly the oracle's slots.  A state
handed over this way decodes exactly as the original does."""
import numpy as np
import pytest
import torch

from gpu_util import requires_gpu
from oracle import seed_handoff as ho
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _np(t):
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def _rand_state(B, H, C, d_k, d_v, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn(B, H, d_k, generator=g)
    U = torch.randn(B, H, C, d_k, generator=g).to(dtype)
    V = torch.randn(B, H, C, d_v, generator=g).to(dtype)
    return a.cuda(), U.cuda(), V.cuda()


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16, torch.float16])
@pytest.mark.parametrize("dims,R,C", [((128, 128), 16, 48), ((128, 64), 16, 16), ((64, 64), 32, 96)])
def test_pack_unpack_bit_exact(dtype, dims, R, C):
    d_k, d_v = dims
    if dtype != torch.float32:
        C = R                   # the 16-bit form's kept arrays hold R columns
    B, H = 6, 5
    a, U, V = _rand_state(B, H, C, d_k, d_v, dtype, 3 + R)
    sel = [4, 0, 9, 5, -2, 2]                 # 9 and -2 select nothing
    hb = binding.handoff_head_bytes(d_k, d_v, R, dtype)
    assert hb == ho.unit_bytes(d_k, d_v, R, 4 if dtype == torch.float32 else 2)
    buf = torch.full((len(sel) * H * hb,), 0xAB, dtype=torch.uint8, device="cuda")
    binding.seed_pack_states(a, U, V, R, torch.tensor(sel, dtype=torch.int32, device="cuda"), buf)
    torch.cuda.synchronize()
    want = ho.pack(_np(a), _np(U), _np(V), R, sel, buf=np.full(buf.numel(), 0xAB, np.uint8))
    assert np.array_equal(buf.cpu().numpy(), want)

    a2, U2, V2 = _rand_state(B, H, C, d_k, d_v, dtype, 50 + R)
    slots = [1, 3, 0, 7, 2, -1]
    ra, rU, rV = ho.unpack(want, _np(a2), _np(U2), _np(V2), R, slots)
    binding.seed_unpack_states(buf, a2, U2, V2, R,
                               torch.tensor(slots, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    assert np.array_equal(_np(a2), ra)
    assert np.array_equal(_np(U2), rU)
    assert np.array_equal(_np(V2), rV)


def test_pack_all_units_of_a_large_batch():
    """256 requests x 32 heads (the 36-layer workload's per-layer launch)."""
    B, H, d_k, d_v, R, C = 256, 32, 128, 128, 16, 48
    a, U, V = _rand_state(B, H, C, d_k, d_v, torch.float32, 9)
    sel = torch.arange(B - 1, -1, -1, dtype=torch.int32, device="cuda")   # reversed order
    buf = torch.empty(B * H * binding.handoff_head_bytes(d_k, d_v, R), dtype=torch.uint8,
                      device="cuda")
    binding.seed_pack_states(a, U, V, R, sel, buf)
    torch.cuda.synchronize()
    got = buf.cpu().numpy()
    an, Un, Vn = _np(a), _np(U), _np(V)
    hb = ho.unit_bytes(d_k, d_v, R)
    for i in (0, 1, 100, B - 1):
        b = B - 1 - i
        want = ho.pack(an[b:b + 1], Un[b:b + 1], Vn[b:b + 1], R, [0])
        assert np.array_equal(got[i * H * hb:(i + 1) * H * hb], want), i


@pytest.mark.parametrize("form", ["in_place", "lazy", "fp16"])
def test_handed_over_state_decodes_identically(form):
    """Prefill -> conversion -> pack on one state; unpack into the slots of a
    second batch; both then decode the same inputs to the same outputs."""
    rule, B, H, d_k, d_v, R, W = "gdn", 4, 8, 128, 128, 16, 32
    vbar = wl.make_vbar(H, d_v, 21, 0, "cuda")
    S = torch.zeros(B, H, d_k, d_v, device="cuda")
    o = torch.empty(B, H, d_v, device="cuda")
    for t in range(-32, 0):
        x = wl.make_step(rule, B, H, d_k, d_v, vbar, 21, t, 0, torch.bfloat16, "cuda")
        binding.dense_decode_step(rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)

    def make():
        if form == "fp16":
            return binding.ShallowState16(rule, B, H, d_k, d_v, R, W, vbar, store=torch.float16)
        return binding.ShallowState(rule, B, H, d_k, d_v, R, W, vbar, lazy=form == "lazy")

    src, dst = make(), make()
    src.from_dense(S)
    dst.from_dense(torch.randn(B, H, d_k, d_v, device="cuda"))    # other requests in the slots
    perm = [2, 0, 3, 1]
    buf = src.pack(torch.arange(B, dtype=torch.int32, device="cuda"))
    dst.unpack(buf, torch.tensor(perm, dtype=torch.int32, device="cuda"))
    o1 = torch.empty(B, H, d_v, device="cuda")
    o2 = torch.empty(B, H, d_v, device="cuda")
    inv = [perm.index(b) for b in range(B)]
    for t in range(W + 4):
        x = wl.make_step(rule, B, H, d_k, d_v, vbar, 22, t, 0, torch.bfloat16, "cuda")
        src.step_and_maybe_compress(x["q"], x["k"], x["v"], x["g"], x["beta"], o1)
        # the same request's inputs, in its new slot
        xp = {k: (None if v is None else v[inv].contiguous()) for k, v in x.items()}
        dst.step_and_maybe_compress(xp["q"], xp["k"], xp["v"], xp["g"], xp["beta"], o2)
        assert torch.equal(o2, o1[inv]), t


@pytest.mark.parametrize("lazy", [False, True])
@pytest.mark.parametrize("rule,dims", [("gdn", (128, 128)), ("kda", (128, 128)),
                                       ("mamba2", (128, 64))])
def test_join_mid_window(rule, dims, lazy):
    """Requests handed over while the batch is k steps into its window join
    it (seed_join_states): each joined slot then follows the oracle started
    from the handed-over state -- its own Lemma 2 steps, then the
    compression of its R + (steps since the join) columns at the batch's
    compression -- and every other slot is bit-identical to a batch that
    saw no join."""
    import numpy as np

    import oracle
    from gpu_util import (TOL_READOUT, TOL_STATE_COMPRESS, TOL_STATE_STEP, f64, inputs_np,
                          rel_err, state_rel_err, true_U)

    d_k, d_v = dims
    B, H, R, W, k_join = 5, 3, 16, 16, 6
    vbar = wl.make_vbar(H, d_v, 61, 0, "cuda")

    def prefilled(seed):
        S = torch.zeros(B, H, d_k, d_v, device="cuda")
        o = torch.empty(B, H, d_v, device="cuda")
        for t in range(-40, 0):
            x = wl.make_step(rule, B, H, d_k, d_v, vbar, seed, t, 0, torch.bfloat16, "cuda")
            binding.dense_decode_step(rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        return S

    def state():
        return binding.ShallowState(rule, B, H, d_k, d_v, R, W, vbar, device="cuda", lazy=lazy)

    S_batch, S_new = prefilled(62), prefilled(63)
    batch, ref = state(), state()
    batch.from_dense(S_batch)
    ref.from_dense(S_batch)
    arrivals = state()
    arrivals.from_dense(S_new)
    src = torch.tensor([1, 3], dtype=torch.int32, device="cuda")     # arriving requests
    slots = torch.tensor([4, 0], dtype=torch.int32, device="cuda")   # their slots in the batch
    buf = arrivals.pack(src)
    o, o_ref = torch.empty(B, H, d_v, device="cuda"), torch.empty(B, H, d_v, device="cuda")
    xs = [wl.make_step(rule, B, H, d_k, d_v, vbar, 64, t, 0, torch.bfloat16, "cuda")
          for t in range(W + 8)]
    for t in range(k_join):
        for st, out in ((batch, o), (ref, o_ref)):
            st.step_and_maybe_compress(xs[t]["q"], xs[t]["k"], xs[t]["v"], xs[t]["g"],
                                       xs[t]["beta"], out)
    batch.join(buf, slots)
    torch.cuda.synchronize()
    assert batch.r == R + k_join
    # the oracle's copy of the joined requests: the handed-over state itself
    units = [int(s) * H + h for s in slots.tolist() for h in range(H)]
    srcu = [int(s) * H + h for s in src.tolist() for h in range(H)]
    vb = np.broadcast_to(f64(vbar)[None], (B, H, d_v)).reshape(-1, d_v)[units]
    a = f64(arrivals.a).reshape(B * H, d_k)[srcu]
    U = f64(arrivals.U).reshape(B * H, -1, d_k)[srcu, :R].transpose(0, 2, 1)
    V = f64(arrivals.V).reshape(B * H, -1, d_v)[srcu, :R].transpose(0, 2, 1)
    others = [u for u in range(B * H) if u not in units]
    compressed = False
    for t in range(k_join, len(xs)):
        x = xs[t]
        c1 = batch.step_and_maybe_compress(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        c2 = ref.step_and_maybe_compress(x["q"], x["k"], x["v"], x["g"], x["beta"], o_ref)
        assert c1 == c2
        xi = {key: (None if val is None else val[units]) for key, val in inputs_np(x).items()}
        a, U, V, o_or = oracle.seed_step(rule, a, U, V, vb, **xi)
        if c1:
            U, V = oracle.compress(U, V, R)
            compressed = True
        og = f64(o).reshape(B * H, d_v)
        assert rel_err(og[units], o_or, -1).max() < TOL_READOUT, t
        assert torch.equal(o.reshape(B * H, d_v)[others], o_ref.reshape(B * H, d_v)[others]), t
        ga = f64(batch.a).reshape(B * H, d_k)[units]
        # the joined slots hold r columns, the first r - (steps since the
        # join) - R of them zero before the compression
        gU = f64(true_U(batch)).reshape(B * H, -1, d_k)[units, :batch.r].transpose(0, 2, 1)
        gV = f64(batch.V).reshape(B * H, -1, d_v)[units, :batch.r].transpose(0, 2, 1)
        tol = TOL_STATE_COMPRESS if compressed else TOL_STATE_STEP
        assert state_rel_err(ga, gU, gV, a, U, V, vb).max() < tol, t
    assert compressed
    for name in ("a", "U", "V") + (("gam",) if lazy else ()):
        x, y = getattr(batch, name), getattr(ref, name)
        assert torch.equal(x.reshape(B * H, -1)[others], y.reshape(B * H, -1)[others]), name
