"""The C ABI without a GPU: libseed.so loads, exports every function that
include/seed.h declares, and rejects bad arguments on the host before any
HIP call (so these run on a machine without a GPU)."""
import ctypes

import pytest

from sink_rank_recurrent_amd import binding

L = binding.lib()
ALIGNED = ctypes.c_void_p(0x10000)     # never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10004)


def test_exports_every_declared_function():
    names = binding.header_functions()
    assert set(names) == {"seed_decode_step", "seed_decode_step_lazy", "seed_compress",
                          "seed_compress_lazy", "seed_state_from_dense", "dense_decode_step",
                          "seed_decode_step_h16", "seed_compress_h16", "seed_round_factors",
                          "seed_handoff_head_bytes", "seed_pack_states", "seed_unpack_states",
                          "seed_state_stats", "seed_stat_fields",
                          "seed_decode_step_sched", "seed_compress_sched", "seed_stream_copy",
                          "seed_status_string", "seed_last_error", "seed_abi_version",
                          "seed_workspace_bytes", "seed_join_states"}
    for n in names:
        assert hasattr(L, n), n
    assert L.seed_abi_version() == 109


def test_status_strings():
    assert L.seed_status_string(0) == b"ok"
    assert L.seed_status_string(4) == b"factor capacity full"
    assert L.seed_status_string(99) == b"unknown status"


def _step(rule=0, batch=2, heads=3, d_k=128, d_v=128, cap=48, r=16, ptr=ALIGNED, beta=ALIGNED,
          dtype=1):
    p = ptr
    return L.seed_decode_step(rule, batch, heads, d_k, d_v, cap, r, p, p, p, p, p, p, p, dtype, p,
                              beta, p, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(r=48), 4, "compress first"),
    (dict(r=49), 2, "r <= cap"),
    (dict(r=-1), 2, "r <= cap"),
    (dict(batch=0), 2, "positive"),
    (dict(d_v=100), 3, "not supported"),
    (dict(d_k=64, d_v=128), 3, "not supported"),
    (dict(cap=128, r=10), 3, "capacity"),
    (dict(rule=7), 1, "unknown rule"),
    (dict(dtype=5), 1, "dtype"),
    (dict(ptr=None), 1, "NULL"),
    (dict(ptr=MISALIGNED), 1, "aligned"),
    (dict(rule=2), 1, "beta must be NULL"),
    (dict(rule=0, beta=None), 1, "beta is NULL"),
])
def test_step_rejects(kwargs, status, needle):
    assert _step(**kwargs) == status
    assert needle in L.seed_last_error().decode()


def test_compress_validation():
    p = ALIGNED
    assert L.seed_compress(1, 1, 128, 128, 48, 48, 0, p, p, None) == 2          # R = 0
    assert L.seed_compress(1, 1, 128, 128, 48, 48, 33, p, p, None) == 3         # R > 32
    assert L.seed_compress(1, 1, 128, 128, 48, 50, 16, p, p, None) == 2         # r > cap
    assert L.seed_compress(1, 1, 128, 128, 48, 48, 16, None, p, None) == 1
    # r <= R is a no-op that touches nothing (pointers are never dereferenced)
    assert L.seed_compress(1, 1, 128, 128, 48, 16, 16, p, p, None) == 0
    assert L.seed_last_error() == b""


def test_lazy_validation():
    p = ALIGNED
    # the lazy step checks what the in-place step checks, and gam
    assert L.seed_decode_step_lazy(0, 2, 3, 128, 128, 48, 48, p, p, p, p, p, p, p, p, 1, p, p, p,
                                   None) == 4
    assert L.seed_decode_step_lazy(0, 2, 3, 128, 128, 48, 16, p, p, p, None, p, p, p, p, 1, p, p,
                                   p, None) == 1
    assert b"gam" in L.seed_last_error()
    assert L.seed_decode_step_lazy(0, 2, 3, 128, 128, 48, 16, p, p, p, MISALIGNED, p, p, p, p, 1,
                                   p, p, p, None) == 1
    assert L.seed_compress_lazy(1, 1, 1, 128, 128, 48, 48, 16, p, p, None, None) == 1
    assert b"gam" in L.seed_last_error()
    assert L.seed_compress_lazy(9, 1, 1, 128, 128, 48, 48, 16, p, p, p, None) == 1
    assert L.seed_compress_lazy(1, 1, 1, 128, 128, 48, 48, 33, p, p, p, None) == 3
    # r <= R: nothing launched, gam untouched
    assert L.seed_compress_lazy(1, 1, 1, 128, 128, 48, 16, 16, p, p, p, None) == 0


def _step_h16(rule=0, R=16, W=32, r=20, store=2, ptr=ALIGNED, gam=ALIGNED, Uk=ALIGNED):
    p = ptr
    return L.seed_decode_step_h16(rule, 2, 3, 128, 128, R, W, r, p, Uk, p, p, p, gam, p, p, p, p,
                                  1, store, p, p, p, None)


@pytest.mark.parametrize("kwargs,status,needle", [
    (dict(r=48), 4, "compress first"),
    (dict(r=15), 2, "R <= r"),
    (dict(r=49), 2, "R <= r"),
    (dict(R=0, r=0), 2, "R > 0"),
    (dict(W=90, r=20), 3, "capacity"),
    (dict(R=12, r=20), 3, "R = 16 or 32"),
    (dict(store=0), 1, "store dtype"),
    (dict(store=3), 1, "store dtype"),
    (dict(gam=None), 1, "gam is NULL"),
    (dict(Uk=MISALIGNED), 1, "Uk is not 16-byte aligned"),
])
def test_step_h16_rejects(kwargs, status, needle):
    assert _step_h16(**kwargs) == status
    assert needle in L.seed_last_error().decode()


def test_compress_h16_and_round_validation():
    p = ALIGNED
    # rule, B, H, d_k, d_v, R, W, r, Uk, Vk, Uw, Vw, gam, store, rounding, seed, epoch, stream
    assert L.seed_compress_h16(0, 1, 1, 128, 128, 16, 32, 48, p, p, p, p, p, 2, 2, 0, 0, None) == 1
    assert b"rounding" in L.seed_last_error()
    assert L.seed_compress_h16(5, 1, 1, 128, 128, 16, 32, 48, p, p, p, p, p, 2, 0, 0, 0, None) == 1
    assert L.seed_compress_h16(0, 1, 1, 128, 128, 33, 32, 48, p, p, p, p, p, 2, 0, 0, 0, None) == 3
    assert L.seed_compress_h16(0, 1, 1, 128, 128, 8, 32, 38, p, p, p, p, p, 2, 0, 0, 0, None) == 3
    assert L.seed_compress_h16(0, 1, 1, 128, 128, 16, 32, 49, p, p, p, p, p, 2, 0, 0, 0, None) == 2
    assert L.seed_compress_h16(0, 1, 1, 128, 128, 16, 32, 48, p, p, p, p, None, 1, 0, 0, 0,
                               None) == 1
    # r == R: nothing to compress, nothing launched
    assert L.seed_compress_h16(0, 1, 1, 128, 128, 16, 32, 16, p, p, p, p, p, 1, 1, 7, 3, None) == 0
    assert L.seed_last_error() == b""
    # B, H, d_k, d_v, R, U, V, Uk, Vk, store, rounding, seed, epoch, stream
    assert L.seed_round_factors(1, 1, 128, 128, 0, p, p, p, p, 1, 0, 0, 0, None) == 2
    assert L.seed_round_factors(1, 1, 128, 128, 16, p, p, p, p, 0, 0, 0, 0, None) == 1
    assert L.seed_round_factors(1, 1, 128, 128, 16, p, p, None, p, 1, 0, 0, 0, None) == 1
    assert L.seed_round_factors(1, 1, 96, 128, 16, p, p, p, p, 1, 0, 0, 0, None) == 3


def test_handoff_validation():
    p = ALIGNED
    assert binding.handoff_head_bytes(128, 128, 16) == 4 * (128 + 256 * 16)
    assert L.seed_handoff_head_bytes(128, 64, 16, 2) == 4 * 128 + 2 * 192 * 16
    assert L.seed_handoff_head_bytes(96, 64, 16, 0) == 0
    # B, H, d_k, d_v, cap, R, store, n_sel, sel, a, U, V, buf, stream
    assert L.seed_pack_states(2, 3, 128, 128, 48, 16, 0, 0, None, None, None, None, None,
                              None) == 0                                  # nothing selected
    assert L.seed_pack_states(2, 3, 128, 128, 48, 16, 0, 2, None, p, p, p, p, None) == 1
    assert L.seed_pack_states(2, 3, 128, 128, 8, 16, 0, 2, p, p, p, p, p, None) == 2   # cap < R
    assert L.seed_pack_states(2, 3, 128, 128, 48, 16, 7, 2, p, p, p, p, p, None) == 1
    assert L.seed_unpack_states(2, 3, 128, 100, 48, 16, 0, 2, p, p, p, p, p, None) == 3
    assert L.seed_unpack_states(2, 3, 128, 128, 48, 16, 0, -1, p, p, p, p, p, None) == 2
    assert L.seed_unpack_states(2, 3, 128, 128, 48, 16, 0, 2, p, p, p, MISALIGNED, p, None) == 1


def test_stats_validation():
    p = ALIGNED
    assert L.seed_stat_fields() == 16
    assert L.seed_state_stats(1, 1, 128, 128, 129, p, p, p, None, None, None) == 2
    assert L.seed_state_stats(1, 1, 128, 96, 16, p, p, p, None, None, None) == 3
    assert L.seed_state_stats(1, 1, 128, 128, 16, p, p, None, None, None, None) == 1
    assert L.seed_state_stats(1, 1, 128, 128, 16, p, p, p, MISALIGNED, None, None) == 1


def test_sched_validation():
    p = ALIGNED
    def step(R=16, W=32, D=8, t_start=p, dtype=1):
        return L.seed_decode_step_sched(0, 2, 3, 128, 128, R, W, D, 5, t_start, p, p, p, p, p, p, p,
                                        p, p, p, p, dtype, p, p, p, None)
    assert step(D=32) == 2 and step(D=-1) == 2 and step(W=0, D=0) == 2
    assert step(R=8) == 3 and step(W=64, D=20) == 3
    assert step(t_start=None) == 1 and step(dtype=3) == 1
    # rule, B, H, d_k, d_v, R, W, D, t_snap, t_start, n, units, KU, KV, Uw, Vw, gam_snap, stream
    assert L.seed_compress_sched(0, 2, 3, 128, 128, 16, 32, 8, 32, p, 0, None, None, None, None,
                                 None, None, None) == 0                      # nothing listed
    assert L.seed_compress_sched(0, 2, 3, 128, 128, 16, 32, 8, 32, p, 7, p, p, p, p, p, p,
                                 None) == 2                                  # more than B*H
    assert L.seed_compress_sched(0, 2, 3, 128, 128, 16, 32, 8, 32, p, 2, None, p, p, p, p, p,
                                 None) == 1


def test_from_dense_validation():
    p = ALIGNED
    assert L.seed_state_from_dense(1, 1, 128, 64, 48, 65, p, p, p, p, p, None) == 2  # R > d_v
    assert L.seed_state_from_dense(1, 1, 128, 128, 16, 17, p, p, p, p, p, None) == 2  # R > cap
    assert L.seed_state_from_dense(1, 1, 128, 128, 48, 33, p, p, p, p, p, None) == 3
    assert L.seed_state_from_dense(1, 1, 128, 128, 48, 16, p, MISALIGNED, p, p, p, None) == 1


def test_dense_step_validation():
    p = ALIGNED
    assert L.dense_decode_step(0, 1, 1, 128, 96, p, p, p, p, 0, p, p, p, None) == 3
    assert L.dense_decode_step(2, 1, 1, 128, 64, p, p, p, p, 0, p, p, p, None) == 1  # beta non-NULL
    assert L.dense_decode_step(1, 1, 1, 128, 128, None, p, p, p, 0, p, p, p, None) == 1


def test_stream_copy_validation():
    a, b = ctypes.c_void_p(0x10000), ctypes.c_void_p(0x20000)
    assert L.seed_stream_copy(a, b, 17, None) == 1                       # not whole vectors
    assert L.seed_stream_copy(a, ctypes.c_void_p(0x10010), 64, None) == 1  # overlapping
    assert b"overlap" in L.seed_last_error()
    assert L.seed_stream_copy(None, b, 64, None) == 1
    assert L.seed_stream_copy(MISALIGNED, b, 64, None) == 1


def test_binding_refuses_host_tensors():
    import torch
    U = torch.zeros(1, 1, 48, 128)
    V = torch.zeros(1, 1, 48, 128)
    with pytest.raises(ValueError, match="device memory"):
        binding.seed_compress(U, V, 48, 16)


def test_scheduled_state_rejects_bad_batching():
    """A snapshot must be compressed before its merge D steps later, so the
    snapshots of at most max(D, 1) steps share a launch; checked before any
    device memory is touched."""
    import torch
    vbar = torch.zeros(2, 128)
    for kw, D in (({"batch_steps": 5}, 4), ({"batch_steps": 2}, 0), ({"batch_steps": 0}, 4),
                  ({"side_streams": -1}, 4), ({}, 16)):
        with pytest.raises(ValueError):
            binding.ScheduledState("gdn", 1, 2, 128, 128, 16, 16, D, vbar, [0], **kw)


def test_workspace_bytes():
    """Every compression and conversion keeps its intermediates on chip: the
    workspace is 0 for every shape they accept, and the query rejects the
    shapes they reject."""
    reject = ctypes.c_size_t(-1).value
    L.seed_workspace_bytes.restype = ctypes.c_size_t
    for d_k, d_v in ((128, 128), (128, 64), (64, 64)):
        for cap, R in ((32, 16), (48, 16), (80, 16), (96, 32), (16, 16)):
            assert L.seed_workspace_bytes(256, 32, d_k, d_v, cap, R) == 0
    assert binding.workspace_bytes(64, 16, 128, 128, 48, 16) == 0
    for args in ((0, 1, 128, 128, 48, 16), (1, 1, 128, 100, 48, 16), (1, 1, 128, 128, 97, 16),
                 (1, 1, 128, 128, 48, 49), (1, 1, 128, 128, 96, 33), (1, 1, 128, 128, 48, 0)):
        assert L.seed_workspace_bytes(*args) == reject, args
    with pytest.raises(ValueError):
        binding.workspace_bytes(1, 1, 128, 100, 48, 16)


def test_join_validation():
    """Joining needs R <= r < cap; nothing selected is a no-op; the lazy
    form's gam is checked only when given.  (No call here passes every
    check: the pointers are not real device memory.)"""
    p = ALIGNED
    fj = L.seed_join_states
    assert fj(0, 4, 2, 128, 128, 48, 16, 15, 1, p, p, p, p, p, None, None) == 2   # r < R
    assert fj(0, 4, 2, 128, 128, 48, 16, 48, 1, p, p, p, p, p, None, None) == 2   # r = cap
    assert fj(5, 4, 2, 128, 128, 48, 16, 20, 1, p, p, p, p, p, None, None) == 1   # rule
    assert fj(0, 4, 2, 128, 128, 48, 16, 20, 1, None, p, p, p, p, None, None) == 1
    assert fj(1, 4, 2, 128, 128, 48, 16, 20, 1, p, p, p, p, p, MISALIGNED, None) == 1
    assert b"gam" in L.seed_last_error()
    assert fj(0, 4, 2, 128, 128, 48, 16, 20, 0, None, None, None, None, None, None, None) == 0
