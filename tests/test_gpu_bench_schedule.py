"""The layer stack bench.py times, on both compression schedules: on the
launch stream after each bench step, and forked onto a side stream right
after the step launch that ends a layer's window and joined right before
that layer's next step launch.  The kernels are deterministic and the layers
independent, so the two runs must leave bit-identical states and read-outs;
a missing wait (a compression still running when its layer steps, or a step
still running when its compression starts) would show as a difference."""
import dataclasses

import pytest
import torch

import bench
from gpu_util import requires_gpu
from sink_rank_recurrent_amd import workloads as wl

pytestmark = [pytest.mark.gpu, requires_gpu]


@pytest.mark.parametrize("form", ["lazy", "in_place"])
def test_overlapped_schedule_equals_launch_stream_order(form):
    # six layers of 8 requests x 8 GDN heads, the 36-layer workload's shapes
    w = dataclasses.replace(wl.WORKLOADS[5], name="gdn_8x8_6L", batch=8, heads=8, layers=6,
                            prefill=64)
    L, dev = w.layers, "cuda"
    spec = bench.Spec(w)
    phases = bench.layer_phases(L, w.W)
    pre, settle, timed = w.W, 8, 2 * w.W
    vbars, Ss = bench.prefill_layers(w, L, dev)
    inputs = bench.make_inputs(w, vbars, pre + settle + timed, dev)
    runs = []
    for overlap in (False, True):
        states, _ = bench.make_states(w, form, vbars, Ss, phases, dev)
        outs = [torch.empty(w.batch, w.heads, w.d_v, device=dev) for _ in range(L)]
        res = bench.run_stack(spec, states, inputs, outs, pre, settle, timed, form, dev,
                              overlap=overlap)
        torch.cuda.synchronize()
        assert res["overlap"] == overlap
        assert res["compressions"] >= L   # every layer compresses in the timed steps
        tensors = []
        for st, o in zip(states, outs):
            tensors += [st.a, st.U, st.V, o] + ([st.gam] if st.gam is not None else [])
        runs.append(([x.clone() for x in tensors], [st.r for st in states]))
    (x0, r0), (x1, r1) = runs
    assert r0 == r1
    for i, (a, b) in enumerate(zip(x0, x1)):
        assert torch.equal(a, b), i
