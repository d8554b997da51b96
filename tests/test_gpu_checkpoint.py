"""Checkpoint and resume of shallow states mid-window.

The state is plain caller-owned device memory (a, U, V; the decay product
gam of the lazy forms; the 16-bit form's kept and window columns) plus the
host integers the binding keeps (the column count r, the window limit and,
for stochastic rounding, the epoch).  A checkpoint is a copy of those to
host bytes; a resume writes them into freshly allocated tensors.  Every
kernel is deterministic (one workgroup per unit, no atomics), so a run
saved mid-window and resumed -- through a compression and into the next
window -- must be bit-identical to the run that never stopped: every
read-out and every final array."""
import io

import numpy as np
import pytest
import torch

from gpu_util import requires_gpu
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]

B, H = 4, 6


def _arrays(st):
    names = ("a", "U", "V", "gam") if isinstance(st, binding.ShallowState) else \
        ("a", "Uk", "Vk", "Uw", "Vw", "gam")
    return {n: getattr(st, n) for n in names if getattr(st, n) is not None}


def _host_ints(st):
    return {"r": st.r, "limit": st.limit, "epoch": getattr(st, "epoch", 0)}


def save(st) -> bytes:
    buf = io.BytesIO()
    arrs = {n: t.detach().cpu().view(torch.int16).numpy() if t.dtype in (torch.float16, torch.bfloat16)
            else t.detach().cpu().numpy() for n, t in _arrays(st).items()}
    np.savez(buf, **arrs, **{f"int_{k}": np.array(v) for k, v in _host_ints(st).items()})
    return buf.getvalue()


def restore(blob: bytes, make):
    st = make()
    z = np.load(io.BytesIO(blob))
    for n, t in _arrays(st).items():
        x = torch.from_numpy(z[n])
        if t.dtype in (torch.float16, torch.bfloat16):
            x = x.view(t.dtype)
        t.copy_(x.to(t.device))
    st.r, st.limit = int(z["int_r"]), int(z["int_limit"])
    if hasattr(st, "epoch"):
        st.epoch = int(z["int_epoch"])
    return st


@pytest.mark.parametrize("form", ["in_place", "lazy", "fp16_stochastic"])
@pytest.mark.parametrize("rule,dims", [("gdn", (128, 128)), ("kda", (128, 128)),
                                       ("mamba2", (128, 64))])
def test_resume_is_bit_identical(form, rule, dims):
    d_k, d_v = dims
    R, W = 16, 16
    vbar = wl.make_vbar(H, d_v, 41, 0, "cuda")

    def make():
        if form == "fp16_stochastic":
            return binding.ShallowState16(rule, B, H, d_k, d_v, R, W, vbar, store=torch.float16,
                                          rounding="stochastic", seed=77, device="cuda")
        return binding.ShallowState(rule, B, H, d_k, d_v, R, W, vbar, device="cuda",
                                    lazy=(form == "lazy"))

    S = torch.zeros(B, H, d_k, d_v, device="cuda")
    o = torch.empty(B, H, d_v, device="cuda")
    for t in range(-40, 0):
        x = wl.make_step(rule, B, H, d_k, d_v, vbar, 42, t, 0, torch.bfloat16, "cuda")
        binding.dense_decode_step(rule, S, x["q"], x["k"], x["v"], x["g"], x["beta"], o)
    xs = [wl.make_step(rule, B, H, d_k, d_v, vbar, 43, t, 0, torch.bfloat16, "cuda")
          for t in range(2 * W + 5)]
    cut = W // 2 + 3                              # mid-window

    ref = make()
    ref.from_dense(S)
    ref_out = []
    blob = None
    for t, x in enumerate(xs):
        if t == cut:
            torch.cuda.synchronize()
            blob = save(ref)
        ref.step_and_maybe_compress(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        ref_out.append(o.clone())
    torch.cuda.synchronize()

    res = restore(blob, make)
    assert res.r == ref.R + cut
    for t in range(cut, len(xs)):
        x = xs[t]
        res.step_and_maybe_compress(x["q"], x["k"], x["v"], x["g"], x["beta"], o)
        assert torch.equal(o, ref_out[t]), t
    torch.cuda.synchronize()
    assert (res.r, res.limit) == (ref.r, ref.limit)
    for n, t in _arrays(ref).items():
        assert torch.equal(_arrays(res)[n], t), n
