"""HIP graphs captured from the C-ABI calls (the way bench.py times the
decode loop) replay bit for bit like the same calls run eagerly.

A window of W decode steps followed by the compression is captured once on
one state; the same calls run eagerly on a copy.  The graph is then
replayed three times, each time from the saved starting state restored by
ordinary eager copies, with synchronisations in between, and every replay's
a, U, V and o must equal the eager result exactly."""
import pytest
import torch

from gpu_util import make_state, requires_gpu
from sink_rank_recurrent_amd import binding
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


def _window(st, inputs, o, r0):
    for t, x in enumerate(inputs):
        binding.seed_decode_step(st.rule, st.a, st.U, st.V, st.vbar, x["q"], x["k"], x["v"],
                                 x["g"], x["beta"], o, r0 + t)
    binding.seed_compress(st.U, st.V, r0 + len(inputs), st.R)


@pytest.mark.parametrize("rule,dims,R,W", [("gdn", (128, 128), 16, 32), ("kda", (128, 128), 16, 64),
                                           ("mamba2", (128, 64), 16, 32)])
def test_graph_replay_matches_eager(rule, dims, R, W):
    d_k, d_v = dims
    B, H = 4, 8
    gen = torch.Generator(device="cuda").manual_seed(90)
    vbar = torch.randn(H, d_v, device="cuda", generator=gen)
    st = make_state(rule, B, H, d_k, d_v, R, W, vbar)
    st.a.copy_(torch.randn(B, H, d_k, device="cuda", generator=gen))
    st.U[:, :, :R] = torch.randn(B, H, R, d_k, device="cuda", generator=gen) / d_k ** 0.5
    st.V[:, :, :R] = torch.randn(B, H, R, d_v, device="cuda", generator=gen)
    inputs = [wl.make_step(rule, B, H, d_k, d_v, vbar, 91, t, 0, torch.bfloat16, "cuda")
              for t in range(W)]
    start = [x.clone() for x in (st.a, st.U, st.V)]
    o = torch.zeros(B, H, d_v, device="cuda")

    # eager reference on a copy of the state
    ref = make_state(rule, B, H, d_k, d_v, R, W, vbar)
    for dst, src in zip((ref.a, ref.U, ref.V), start):
        dst.copy_(src)
    o_ref = torch.zeros_like(o)
    _window(ref, inputs, o_ref, R)
    torch.cuda.synchronize()

    # warm-up eager window (first calls set kernel attributes), then capture
    _window(st, inputs, o, R)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _window(st, inputs, o, R)
    torch.cuda.synchronize()
    for rep in range(3):
        for dst, src in zip((st.a, st.U, st.V), start):
            dst.copy_(src)
        o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(st.a, ref.a), rep
        assert torch.equal(st.U[:, :, :R], ref.U[:, :, :R]), rep
        assert torch.equal(st.V[:, :, :R], ref.V[:, :, :R]), rep
        assert torch.equal(o, o_ref), rep
