"""Pins of the oracle's 16-bit factor storage (oracle/seed_rounding.py).

The generator is pinned by the published known-answer vectors of
Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers: As Easy
as 1, 2, 3", SC 2011; the vectors distributed with the authors' Random123
library).  Nearest rounding is pinned against two independent conversions
(numpy's fp32 -> fp16 and torch's fp32 -> bf16, both round-to-nearest-even),
stochastic rounding by its defining probability, counted exactly over all
2^24 values of u, and the rounded compression by the rounding bound.
"""
import numpy as np
import pytest
import torch

from oracle import seed_oracle as so
from oracle import seed_rounding as rd

# (counter, key) -> words, Philox4x32-10 known answers
KAT = [
    ((0, 0, 0, 0), (0, 0), (0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8)),
    ((0xFFFFFFFF,) * 4, (0xFFFFFFFF,) * 2, (0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD)),
    ((0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344), (0xA4093822, 0x299F31D0),
     (0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1)),
]


@pytest.mark.parametrize("ctr,key,want", KAT)
def test_philox_known_answers(ctr, key, want):
    got = rd.philox4x32_10(np.array(ctr), np.array(key))
    assert tuple(int(x) for x in got) == want


def _probe_values(rng, n=20000):
    """fp32 values over the whole fp16 range and beyond: log-uniform
    magnitudes, both signs, the subnormal range, the overflow edge, zeros."""
    mag = np.exp2(rng.uniform(-30.0, 18.0, n))
    x = (mag * rng.choice([-1.0, 1.0], n)).astype(np.float32)
    edge = np.array([0.0, -0.0, 65504.0, 65519.99, 65520.0, 65535.0, 65536.0, 1e6,
                     2.0 ** -24, 2.0 ** -25, 1.5 * 2.0 ** -25, 2.0 ** -26, 6e-8, 2.0 ** -14,
                     2.0 ** -14 - 2.0 ** -25, 3.0e38, 1e-40], dtype=np.float32)
    return np.concatenate([x, edge, -edge])


def _fp16_ties(rng, n=4000):
    """Values exactly halfway between adjacent fp16 numbers (normal and
    subnormal), both parities of the lower neighbour."""
    b = rng.integers(1, 0x7BFF, n).astype(np.uint16)
    lo = b.view(np.float16).astype(np.float64)
    hi = (b + 1).view(np.float16).astype(np.float64)
    return ((lo + hi) / 2).astype(np.float32)


def test_nearest_fp16_matches_numpy():
    rng = np.random.default_rng(1)
    x = np.concatenate([_probe_values(rng), _fp16_ties(rng)])
    x = np.concatenate([x, -x])
    with np.errstate(over="ignore"):
        want = x.astype(np.float16).view(np.uint16)
    got = rd.round_nearest(x, rd.FP16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_nearest_bf16_matches_torch():
    rng = np.random.default_rng(2)
    mag = np.exp2(rng.uniform(-140.0, 127.9, 30000))
    x = (mag * rng.choice([-1.0, 1.0], mag.size)).astype(np.float32)
    # exact ties: the low 16 bits of an fp32 pattern equal to 0x8000
    tb = (rng.integers(0, 0x7F7F, 4000).astype(np.uint32) << 16) | np.uint32(0x8000)
    x = np.concatenate([x, tb.view(np.float32), -tb.view(np.float32),
                        np.array([0.0, -0.0, 3.3895314e38, 3.4028235e38, 1e-42], np.float32)])
    want = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = rd.round_nearest(x, rd.BF16)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(x[i]), hex(got[i]), hex(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("fmt", [rd.BF16, rd.FP16])
def test_stochastic_returns_a_neighbour(fmt):
    rng = np.random.default_rng(3)
    x = _probe_values(rng)
    x = x[np.abs(x) < (60000.0 if fmt == rd.FP16 else 1e38)]
    words = rng.integers(0, 2 ** 32, x.size, dtype=np.uint64).astype(np.uint32)
    got = rd.widen(rd.round_stochastic(x, fmt, words), fmt)
    dn = rd.widen(rd.round_stochastic(x, fmt, np.full(x.size, 0xFFFFFFFF, np.uint32)), fmt)
    up = rd.widen(rd.round_stochastic(x, fmt, np.zeros(x.size, np.uint32)), fmt)
    xs = x.astype(np.float64)
    # u = max rounds toward zero, u = 0 away from zero unless exact
    assert np.all(np.abs(dn) <= np.abs(xs)) and np.all(np.abs(up) >= np.abs(xs))
    assert np.all((got == dn) | (got == up))
    # the two neighbours are adjacent: nothing of the format lies strictly between
    near = rd.widen(rd.round_nearest(x, fmt), fmt)
    assert np.all((near == dn) | (near == up))
    assert np.all(np.sign(got[got != 0]) == np.sign(xs[got != 0]))


@pytest.mark.parametrize("fmt", [rd.BF16, rd.FP16])
def test_stochastic_keeps_representable_values(fmt):
    rng = np.random.default_rng(4)
    b = rng.integers(0, 0x7C00 if fmt == rd.FP16 else 0x7F80, 5000).astype(np.uint16)
    b = np.concatenate([b, b | np.uint16(0x8000)])
    x = rd.widen(b, fmt).astype(np.float32)
    words = rng.integers(0, 2 ** 32, x.size, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(rd.widen(rd.round_stochastic(x, fmt, words), fmt),
                          rd.widen(b, fmt))


@pytest.mark.parametrize("fmt,x,frac", [
    (rd.FP16, 1.0 + 0.25 * 2.0 ** -10, 0.25),
    (rd.FP16, -(3.0 + 0.6875 * 2.0 ** -9), 0.6875),
    (rd.FP16, 0.3 * 2.0 ** -24, None),            # below the smallest subnormal
    (rd.FP16, 65504.0 + 0.5 * 32.0, 0.5),          # rounds up to infinity half the time
    (rd.BF16, 1.0 + 0.125 * 2.0 ** -7, 0.125),
    (rd.BF16, -(2.0 ** 100) * (1.0 + 0.9375 * 2.0 ** -7), 0.9375),
])
def test_stochastic_probability_is_exact(fmt, x, frac):
    """Over all 2^24 values of u the number of round-ups is (|x|-lo)/(hi-lo)
    2^24, rounded up: the expectation of the rounded value is x up to 2^-24
    of one spacing."""
    x32 = np.float32(x)
    a = abs(float(x32))
    if frac is None:
        frac = a / 2.0 ** -24
    u = np.arange(2 ** 24, dtype=np.uint32) << 8
    got = rd.round_stochastic(np.full(u.size, x32), fmt, u)
    lo_bits = rd.round_stochastic(np.array([x32]), fmt, np.array([0xFFFFFFFF], np.uint32))[0]
    ups = int(np.count_nonzero(got != lo_bits))
    assert ups == int(np.ceil(frac * 2 ** 24))


def test_stochastic_mean_over_philox_words():
    """Unbiased on average over generator words (a statistical check of the
    generator and the rounding together: 4 sigma)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(64) * 0.01).astype(np.float32)
    wU, _ = rd.factor_words(7, 64, 4096, 4, seed=12345, epoch=3)     # 4096 x 64 words
    vals = rd.widen(rd.round_stochastic(np.broadcast_to(x, (4096, 64)), rd.BF16, wU), rd.BF16)
    lo, sp = rd._grid(np.abs(x.astype(np.float64)), rd.BF16)
    p = (np.abs(x) - lo) / sp
    sd = sp * np.sqrt(p * (1 - p) / 4096) + 1e-30
    assert np.all(np.abs(vals.mean(axis=0) - x) <= 4 * sd + 1e-12 * np.abs(x))


def test_factor_words_layout():
    """Every element of a unit's block has its own word; the words depend on
    the unit, the epoch and the seed; U's block comes first."""
    R, d_k, d_v = 4, 8, 12
    wU, wV = rd.factor_words(3, R, d_k, d_v, seed=(5 << 32) | 9, epoch=2)
    assert wU.shape == (d_k, R) and wV.shape == (d_v, R)
    allw = np.concatenate([wU.T.ravel(), wV.T.ravel()])
    assert np.unique(allw).size == allw.size
    # element f = 0 is word 0 of the first counter block
    w0 = rd.philox4x32_10(np.array([0, 3, 2, 0]), np.array([9, 5]))
    assert wU[0, 0] == w0[0] and wU[1, 0] == w0[1] and wU[3, 0] == w0[3]
    for other in (rd.factor_words(4, R, d_k, d_v, (5 << 32) | 9, 2),
                  rd.factor_words(3, R, d_k, d_v, (5 << 32) | 9, 1),
                  rd.factor_words(3, R, d_k, d_v, (6 << 32) | 9, 2)):
        assert np.all(other[0] != wU)


@pytest.mark.parametrize("fmt,mode", [(rd.BF16, rd.NEAREST), (rd.FP16, rd.NEAREST),
                                      (rd.BF16, rd.STOCHASTIC), (rd.FP16, rd.STOCHASTIC)])
def test_compress_rounded_bound(fmt, mode):
    """The stored factors are the truncation's factors within one rounding:
    half a spacing (nearest) or one spacing (stochastic) per element, and
    the rounded state lies within the corresponding bound of the truncation."""
    rng = np.random.default_rng(6)
    d_k, d_v, n, R = 32, 24, 12, 5
    U = rng.standard_normal((d_k, n))
    V = rng.standard_normal((d_v, n)) * 0.3
    Ub, Vb, L, F = rd.compress_rounded(U, V, R, fmt, mode, seed=11, epoch=1, unit=2)
    L2, F2 = so.compress(U, V, R)
    assert np.allclose(L @ F.T, L2 @ F2.T)
    lim = 0.5 if mode == rd.NEAREST else 1.0
    for bits, X in ((Ub, L), (Vb, F)):
        x32 = X.astype(np.float32).astype(np.float64)
        _, sp = rd._grid(np.abs(x32), fmt)
        assert np.all(np.abs(rd.widen(bits, fmt) - x32) <= lim * sp)
    # per element |rd(x) - x| <= lim spacing <= u |x|, u = lim 2^(1-p), plus
    # the step from fp64 to fp32 (2^-24 |x|)
    p = 8 if fmt == rd.BF16 else 11
    u = lim * 2.0 ** (1 - p) + 2.0 ** -24
    Ur, Vr = rd.widen(Ub, fmt), rd.widen(Vb, fmt)
    err = np.linalg.norm(Ur @ Vr.T - L @ F.T)
    assert err <= (2 * u + u * u) * np.linalg.norm(np.abs(L) @ np.abs(F).T)


def test_h16_state_bytes():
    """Right after a compression the 16-bit form holds the fp32 sink
    coefficient and half the factor bytes of the fp32 form."""
    for d_k, d_v, R in ((128, 128, 16), (128, 64, 16), (64, 64, 32)):
        full = so.shallow_state_bytes(d_k, d_v, R, 0)
        half = rd.shallow_state_bytes_h16(d_k, d_v, R, 0)
        assert full - half == 2 * (d_k + d_v) * R
        # appended columns are fp32 in both forms
        assert (rd.shallow_state_bytes_h16(d_k, d_v, R, 5) - half
                == so.shallow_state_bytes(d_k, d_v, R, 5) - full)
