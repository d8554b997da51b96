"""CPU oracle for the shallow-form state handoff (numpy, byte layout).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests use it.  It shares no code with the HIP
library.

At the end of the prefill each state is compressed to the sink plus rank-R
factors (SEED figures and tables on thelatestinai.com, Fig. 1 (a) caption
and Table 1), and a state in that form is what a decode server receives:
the sink coefficient a and R columns of U and V, 4 [d_k + (d_k + d_v) R]
bytes per head in fp32 (the byte account of Table 17 at w = 0), half the
factor bytes with 16-bit factors (Table 4, Table 9).

Reading of what the pages leave open: the handoff unit is one request with
all its heads of a layer.  A packed buffer holds the selected requests one
after another; a request holds its H heads in order; a head holds
  a [d_k] fp32, then U's R columns [R][d_k], then V's R columns [R][d_v],
the factors in the state's storage type (fp32, or the 16-bit patterns of
the 16-bit form).  Unpacking writes a request's heads into a chosen batch
slot; the state then holds r = R columns (and a decay product of 1).
Indices outside [0, batch) select nothing: their part of the buffer (pack)
or their slot (unpack) is left as it was.

Pins: tests/test_oracle_handoff.py (round trip, the byte account of Table 2
and Table 17, placement of every field).
"""
from __future__ import annotations

import numpy as np


def unit_bytes(d_k, d_v, R, factor_bytes=4):
    """Bytes of one packed head: fp32 a, then the R factor columns."""
    return 4 * d_k + factor_bytes * (d_k + d_v) * R


def pack(a, U, V, R, sel, buf=None):
    """Pack requests `sel` of a state into one buffer (uint8).

    a [B, H, d_k] float32; U [B, H, C, d_k], V [B, H, C, d_v] in the storage
    dtype (float32, or uint16 patterns), C >= R columns of which the first R
    are packed.  Returns the buffer: len(sel) requests, each H heads of
    unit_bytes.  If `buf` is given, entries of `sel` outside [0, B) leave
    their part of it unchanged."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    B, H, d_k = a.shape
    d_v = V.shape[-1]
    fb = U.dtype.itemsize
    ub = unit_bytes(d_k, d_v, R, fb)
    out = np.zeros(len(sel) * H * ub, np.uint8) if buf is None else buf.copy()
    for i, b in enumerate(sel):
        if not 0 <= b < B:
            continue
        for h in range(H):
            head = np.concatenate([
                a[b, h].view(np.uint8),
                np.ascontiguousarray(U[b, h, :R]).view(np.uint8).ravel(),
                np.ascontiguousarray(V[b, h, :R]).view(np.uint8).ravel()])
            off = (i * H + h) * ub
            out[off: off + ub] = head
    return out


def unpack(buf, a, U, V, R, slots):
    """Unpack a buffer of len(slots) requests into batch slots `slots`.

    a, U, V as for pack (copies are returned; the inputs are not modified);
    U and V receive columns 0..R-1 of each unpacked head."""
    a, U, V = a.copy(), U.copy(), V.copy()
    B, H, d_k = a.shape
    d_v = V.shape[-1]
    fb = U.dtype.itemsize
    ub = unit_bytes(d_k, d_v, R, fb)
    buf = np.asarray(buf, np.uint8)
    for i, b in enumerate(slots):
        if not 0 <= b < B:
            continue
        for h in range(H):
            off = (i * H + h) * ub
            a[b, h] = buf[off: off + 4 * d_k].view(np.float32)
            off += 4 * d_k
            U[b, h, :R] = buf[off: off + fb * d_k * R].view(U.dtype).reshape(R, d_k)
            off += fb * d_k * R
            V[b, h, :R] = buf[off: off + fb * d_v * R].view(V.dtype).reshape(R, d_v)
    return a, U, V
