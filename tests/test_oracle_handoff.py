"""Pins of the handoff oracle (oracle/seed_handoff.py): the packed size is
the byte account of the pages (Table 17 at w = 0; Table 2's printed state
sizes through the golden file), every field lands where the layout says,
and unpack inverts pack."""
import json
import os

import numpy as np
import pytest

from oracle import seed_handoff as ho
from oracle import seed_oracle as so
from oracle import seed_rounding as rd

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "table2_state_bytes.json")


@pytest.mark.parametrize("d_k,d_v,R", [(128, 128, 16), (128, 64, 16), (64, 64, 32)])
def test_packed_size_is_the_shallow_state_at_w0(d_k, d_v, R):
    assert ho.unit_bytes(d_k, d_v, R, 4) == so.shallow_state_bytes(d_k, d_v, R, 0)
    assert ho.unit_bytes(d_k, d_v, R, 2) == rd.shallow_state_bytes_h16(d_k, d_v, R, 0)


def test_packed_size_against_table2():
    """A request's handoff is its state right after a compression: Table 2's
    'State at R' row (through the golden file that cites it).  Where the
    head count is not printed it follows from the dense size."""
    g = json.load(open(GOLDEN))
    for m in g["models"]:
        heads = m["heads"] or round(m["dense_MB"] * 1e6 / (4 * m["d_k"] * m["d_v"]))
        packed = heads * ho.unit_bytes(m["d_k"], m["d_v"], m["R"], 4) / 1e6
        # printed to 0.1 MB; a head count derived from a rounded dense size
        # adds its own share of the rounding
        slack = 0.05 + (0 if m["heads"] else 0.05 * packed / m["dense_MB"] + 0.01 * packed)
        assert abs(packed - m["at_R_MB"]) <= slack, (m["name"], packed, m["at_R_MB"])


def _state(B, H, C, d_k, d_v, dtype, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((B, H, d_k)).astype(np.float32)
    if dtype == np.float32:
        U = rng.standard_normal((B, H, C, d_k)).astype(np.float32)
        V = rng.standard_normal((B, H, C, d_v)).astype(np.float32)
    else:
        U = rng.integers(0, 1 << 16, (B, H, C, d_k)).astype(np.uint16)
        V = rng.integers(0, 1 << 16, (B, H, C, d_v)).astype(np.uint16)
    return a, U, V


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_fields_land_where_the_layout_says(dtype):
    B, H, C, d_k, d_v, R = 5, 3, 7, 8, 4, 2
    a, U, V = _state(B, H, C, d_k, d_v, dtype, 1)
    sel = [3, 0, 4]
    buf = ho.pack(a, U, V, R, sel)
    fb = np.dtype(dtype).itemsize
    ub = 4 * d_k + fb * (d_k + d_v) * R
    assert buf.size == len(sel) * H * ub
    # request 1 of the buffer is batch slot 0; its head 2 starts at (1*H + 2) ub
    off = (1 * H + 2) * ub
    assert np.array_equal(buf[off: off + 4 * d_k].view(np.float32), a[0, 2])
    u_col1 = buf[off + 4 * d_k + fb * d_k: off + 4 * d_k + 2 * fb * d_k].view(dtype)
    assert np.array_equal(u_col1, U[0, 2, 1])
    v_col0 = buf[off + 4 * d_k + fb * d_k * R: off + 4 * d_k + fb * d_k * R + fb * d_v].view(dtype)
    assert np.array_equal(v_col0, V[0, 2, 0])


@pytest.mark.parametrize("dtype", [np.float32, np.uint16])
def test_unpack_inverts_pack_and_skips_bad_indices(dtype):
    B, H, C, d_k, d_v, R = 6, 2, 5, 8, 8, 3
    a, U, V = _state(B, H, C, d_k, d_v, dtype, 2)
    sel = [5, 1, 2]
    buf = ho.pack(a, U, V, R, sel)
    a2, U2, V2 = _state(B, H, C, d_k, d_v, dtype, 3)
    slots = [0, 4, 9]                    # 9 is outside the batch: nothing written
    ra, rU, rV = ho.unpack(buf, a2, U2, V2, R, slots)
    for src, dst in ((5, 0), (1, 4)):
        assert np.array_equal(ra[dst], a[src])
        assert np.array_equal(rU[dst, :, :R], U[src, :, :R])
        assert np.array_equal(rV[dst, :, :R], V[src, :, :R])
        # columns beyond R are not part of the handoff
        assert np.array_equal(rU[dst, :, R:], U2[dst, :, R:])
    for b in (1, 2, 3, 5):
        assert np.array_equal(ra[b], a2[b]) and np.array_equal(rU[b], U2[b])
    # a pack with an index outside the batch leaves that part of the buffer
    fill = np.full(buf.size, 0xAB, np.uint8)
    out = ho.pack(a, U, V, R, [5, -1, 2], buf=fill)
    ub = buf.size // (3 * H)
    assert np.all(out[H * ub: 2 * H * ub] == 0xAB)
    assert np.array_equal(out[:H * ub], buf[:H * ub])
