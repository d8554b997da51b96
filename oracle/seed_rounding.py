"""CPU oracle for 16-bit factor storage (fp64/integer numpy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
run this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it.  It shares no code with the HIP library.

What the pages fix (SEED figures and tables on thelatestinai.com, Table 4
and its caption; Table 9 and its caption; the picx.dev summary's list of
results, on 16-bit factors halving the state bytes): the shallow state's
factors can be held in fp16 (or bf16), rounded to nearest or stochastically
at every compression.

Readings of what they leave open (each repeated where it is used):
  * "rounded at every compression": the R columns a compression produces
    are rounded once, when they are written, and then kept in 16 bits; the
    columns appended between two compressions are held in fp32 until the
    next compression consumes them, so nothing else is ever rounded.  The
    sink coefficient a and the decay product stay fp32.
  * the value rounded is the fp32 result of the compression: both sides
    take the rounding decision in fp32, from the same kind of value.
  * nearest is IEEE round-to-nearest, ties to the even pattern; values at
    or beyond the format's overflow threshold become infinity.
  * stochastic: a value x between adjacent representable magnitudes
    lo <= |x| < hi is rounded to hi with probability (|x| - lo)/(hi - lo),
    decided by u = (w >> 8) 2^-24 from one 32-bit random word w: up iff
    (|x| - lo)/(hi - lo) > u.  Every quantity in that comparison is exact.
  * the random words are those of the counter-based generator
    Philox4x32-10 (J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw,
    "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): element f of a
    unit's factor block (f = c d_k + i for U[i, c], R d_k + c d_v + i for
    V[i, c]) takes word f mod 4 of Philox(counter = (f div 4, unit, epoch,
    0), key = (seed mod 2^32, seed div 2^32)).

Pins: tests/test_oracle_rounding.py checks the generator against its
published known-answer vectors, nearest rounding against numpy's fp16 and
torch's bf16 conversions, and stochastic rounding against its exact
up-probability by enumeration of all 2^24 values of u.
"""
from __future__ import annotations

import numpy as np

from .seed_oracle import compress

BF16, FP16 = "bf16", "fp16"
NEAREST, STOCHASTIC = "nearest", "stochastic"

# significand bits (with the implicit one), smallest normal exponent,
# largest exponent
_FMT = {BF16: (8, -126, 127), FP16: (11, -14, 15)}

# ---------------------------------------------------------------------------
# Philox4x32-10 (Salmon et al., SC 2011): a 4 x 32-bit counter and a 2 x
# 32-bit key; ten rounds of two 32 x 32 -> 64-bit products, the key bumped
# by the Weyl constants between rounds.
# ---------------------------------------------------------------------------

_M0, _M1 = 0xD2511F53, 0xCD9E8D57
_W0, _W1 = 0x9E3779B9, 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)


def philox4x32_10(ctr, key):
    """ctr [..., 4], key [..., 2] (values < 2^32) -> [..., 4] uint32 words."""
    ctr = np.asarray(ctr, dtype=np.uint64)
    key = np.asarray(key, dtype=np.uint64)
    c0, c1, c2, c3 = (ctr[..., i] for i in range(4))
    k0, k1 = key[..., 0], key[..., 1]
    for rnd in range(10):
        if rnd:
            k0 = (k0 + np.uint64(_W0)) & _MASK
            k1 = (k1 + np.uint64(_W1)) & _MASK
        p0 = np.uint64(_M0) * c0          # < 2^64: no wrap in uint64
        p1 = np.uint64(_M1) * c2
        c0, c1, c2, c3 = ((p1 >> np.uint64(32)) ^ c1 ^ k0, p1 & _MASK,
                          (p0 >> np.uint64(32)) ^ c3 ^ k1, p0 & _MASK)
    return np.stack([c0, c1, c2, c3], axis=-1).astype(np.uint32)


def factor_words(unit, R, d_k, d_v, seed, epoch):
    """The random words of one unit's factor block (reading above).

    Returns (wU [d_k, R], wV [d_v, R]) uint32, wU[i, c] for element
    f = c d_k + i and wV[i, c] for f = R d_k + c d_v + i.
    """
    total = R * (d_k + d_v)
    f = np.arange(total, dtype=np.uint64)
    ctr = np.stack([f // 4, np.full_like(f, unit), np.full_like(f, epoch), np.zeros_like(f)],
                   axis=-1)
    key = np.array([seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF], dtype=np.uint64)
    words = philox4x32_10(ctr, np.broadcast_to(key, ctr.shape[:-1] + (2,)))
    w = words[np.arange(total), (f % 4).astype(np.int64)]
    wU = w[: R * d_k].reshape(R, d_k).T
    wV = w[R * d_k:].reshape(R, d_v).T
    return wU, wV


# ---------------------------------------------------------------------------
# 16-bit rounding of fp32 values, written from the formats' grids
# ---------------------------------------------------------------------------

def _grid(a, fmt):
    """For magnitudes a >= 0 (fp32 values held in fp64): the representable
    neighbours lo <= a < hi = lo + spacing of the format (hi may exceed
    the largest finite value: it then stands for infinity)."""
    p, emin, _ = _FMT[fmt]
    _, ex = np.frexp(a)                    # a = m 2^ex, m in [0.5, 1)
    e = np.maximum(ex - 1, emin)           # exponent of the binade (subnormals: emin)
    spacing = np.ldexp(1.0, e - (p - 1))
    lo = np.floor(a / spacing) * spacing   # exact: scaling by powers of two
    return lo, spacing


def _encode(val, neg, fmt):
    """Bit patterns of representable values val >= 0 (inf above the largest
    finite value) with sign neg."""
    p, _, emax = _FMT[fmt]
    maxf = (2.0 - 2.0 ** (1 - p)) * 2.0 ** emax
    val = np.where(val > maxf, np.inf, val)
    if fmt == FP16:
        bits = val.astype(np.float16).view(np.uint16).astype(np.uint32)   # exact: representable
    else:
        bits = val.astype(np.float32).view(np.uint32) >> 16               # exact: low half zero
    return np.where(neg, bits | np.uint32(0x8000), bits).astype(np.uint16)


def _split(x32):
    x = np.asarray(x32, dtype=np.float32).astype(np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("the oracle rounds finite values only")
    return np.abs(x), np.signbit(x)


def round_nearest(x32, fmt):
    """fp32 -> 16-bit pattern, nearest with ties to the even pattern."""
    a, neg = _split(x32)
    lo, sp = _grid(a, fmt)
    frac = (a - lo) / sp                   # exact
    lo_bits = _encode(lo, np.zeros_like(neg), fmt)
    tie_up = (lo_bits & 1) == 1
    up = (frac > 0.5) | ((frac == 0.5) & tie_up)
    return _encode(np.where(up, lo + sp, lo), neg, fmt)


def round_stochastic(x32, fmt, words):
    """fp32 -> 16-bit pattern, up in magnitude iff (|x| - lo)/(hi - lo) > u,
    u = (w >> 8) 2^-24 for the 32-bit word w of the element."""
    a, neg = _split(x32)
    lo, sp = _grid(a, fmt)
    frac = (a - lo) / sp
    u = (np.asarray(words, dtype=np.uint32) >> 8).astype(np.float64) * 2.0 ** -24
    return _encode(np.where(frac > u, lo + sp, lo), neg, fmt)


def widen(bits, fmt):
    """16-bit patterns -> their exact values (fp64)."""
    b = np.asarray(bits, dtype=np.uint16)
    if fmt == FP16:
        return b.view(np.float16).astype(np.float64)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# The rounded factor block and the compression that produces it
# ---------------------------------------------------------------------------

def round_factors(U32, V32, fmt, mode, seed=0, epoch=0, unit=0):
    """Round one unit's rank-R factors U [d_k, R], V [d_v, R] (fp32 values)
    to 16-bit patterns (reading above); returns (U bits, V bits)."""
    U32 = np.asarray(U32, dtype=np.float32)
    V32 = np.asarray(V32, dtype=np.float32)
    if mode == NEAREST:
        return round_nearest(U32, fmt), round_nearest(V32, fmt)
    if mode != STOCHASTIC:
        raise ValueError(f"unknown rounding {mode!r}")
    wU, wV = factor_words(unit, U32.shape[-1], U32.shape[0], V32.shape[0], seed, epoch)
    return round_stochastic(U32, fmt, wU), round_stochastic(V32, fmt, wV)


def compress_rounded(U, V, R, fmt, mode, seed=0, epoch=0, unit=0):
    """Compression to rank R with the result stored in 16 bits.

    The content U V^T (U at true scale, [d_k, n]; V [d_v, n]) is replaced by
    its rank-R truncation (the oracle's compress: U' orthonormal, V' with
    the singular values); U' and V' are taken to fp32 and rounded to the
    16-bit format (reading above).  Returns (U' bits, V' bits, U' fp64,
    V' fp64): the patterns and the unrounded factors they come from.
    """
    L, F = compress(U, V, R)
    Ub, Vb = round_factors(L.astype(np.float32), F.astype(np.float32), fmt, mode,
                           seed, epoch, unit)
    return Ub, Vb, L, F


def shallow_state_bytes_h16(d_k, d_v, R, w):
    """Bytes of one shallow head state w steps after a compression with
    16-bit kept factors: fp32 sink coefficient, 2-byte R kept columns,
    4-byte columns appended since the compression (the byte account of
    Table 17 of the SEED figures and tables with the kept factors at
    2 bytes)."""
    return 4 * d_k + 2 * (d_k + d_v) * R + 4 * (d_k + d_v) * w
