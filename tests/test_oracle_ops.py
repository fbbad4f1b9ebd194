"""Pins of the oracle's elementwise ops against exact rational arithmetic,
high-precision exp, glibc's fmaf and closed forms."""
import ctypes
import ctypes.util
import math
from fractions import Fraction

import mpmath
import numpy as np
import pytest

from oracle import ops


def round_exact(q: Fraction, dtype) -> np.generic:
    """Nearest value of ``dtype`` to the rational q, ties to even (by exact comparison)."""
    dtype = np.dtype(dtype).type
    c = dtype(float(q))
    cands = {c, np.nextafter(c, dtype(np.inf)), np.nextafter(c, dtype(-np.inf))}
    best = None
    for v in cands:
        if not np.isfinite(v):
            continue
        d = abs(Fraction(float(v)) - q)
        key = (d, int(np.array(v).view(np.uint16 if dtype == np.float16 else np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, v)
    return best[1]


def _rand_f32(rng, n, lo_exp=-30, hi_exp=30):
    m = rng.uniform(1, 2, n)
    e = rng.integers(lo_exp, hi_exp, n)
    s = rng.choice([-1.0, 1.0], n)
    return (s * m * np.exp2(e)).astype(np.float32)


def test_fma_f32_exact_rational():
    rng = np.random.default_rng(11)
    a, x = _rand_f32(rng, 3000), _rand_f32(rng, 3000)
    b = (-(a.astype(np.float64) * x) * rng.uniform(0.5, 1.5, 3000)).astype(np.float32)  # heavy cancellation
    got = ops.fma(a, x, b, np.float32)
    for ai, xi, bi, gi in zip(a, x, b, got):
        q = Fraction(float(ai)) * Fraction(float(xi)) + Fraction(float(bi))
        assert gi == round_exact(q, np.float32) or (q == 0 and gi == 0)


def test_fma_f32_vs_libm_fmaf():
    libm = ctypes.CDLL(ctypes.util.find_library("m"))
    libm.fmaf.restype = ctypes.c_float
    libm.fmaf.argtypes = [ctypes.c_float] * 3
    rng = np.random.default_rng(12)
    a, x, b = (rng.standard_normal(20000).astype(np.float32) for _ in range(3))
    got = ops.fma(a, x, b, np.float32)
    ref = np.array([libm.fmaf(float(p), float(q), float(r)) for p, q, r in zip(a, x, b)], dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_fma_special_cases():
    x = np.float32(1.2345678)
    b = np.float32(-3.5)
    assert ops.fma(np.float32(0), x, b) == b                   # 0 * x + b = b
    assert ops.fma(np.float32(1), x, np.float32(-0.0)) == x    # 1 * x - 0 = x
    # a denormal result survives (no flush to zero)
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    assert ops.fma(np.float32(0.5), np.float32(4) * tiny, np.float32(0)) == np.float32(2) * tiny
    # a case where mul-then-add double-rounds but fma does not: (1 + 2^-12)^2 - 1
    a = np.float32(1 + 2.0 ** -12)
    assert ops.fma(a, a, np.float32(-1)) == np.float32(2.0 ** -11 + 2.0 ** -24)


def test_fma_f16_exact_rational():
    rng = np.random.default_rng(13)
    a, x, b = (rng.standard_normal(3000).astype(np.float16) for _ in range(3))
    got = ops.fma(a, x, b, np.float16)
    for ai, xi, bi, gi in zip(a, x, b, got):
        q = Fraction(float(ai)) * Fraction(float(xi)) + Fraction(float(bi))
        assert gi == round_exact(q, np.float16) or (q == 0 and gi == 0)


def test_add_mul_exact_rational():
    rng = np.random.default_rng(14)
    a, b = _rand_f32(rng, 2000), _rand_f32(rng, 2000, -5, 5)
    s, m = ops.add(a, b), ops.mul(a, b)
    for ai, bi, si, mi in zip(a, b, s, m):
        fa, fb = Fraction(float(ai)), Fraction(float(bi))
        assert si == round_exact(fa + fb, np.float32) or (fa + fb == 0 and si == 0)
        assert mi == round_exact(fa * fb, np.float32)


def test_sqrt_correctly_rounded():
    # correct rounding: the exact root lies between the midpoints to r's neighbours
    rng = np.random.default_rng(15)
    xs = (rng.random(5000, dtype=np.float32) * np.float32(1e4)).astype(np.float32)
    got = ops.sqrt(xs, np.float32)
    for x, r in zip(xs, got):
        lo = np.nextafter(r, np.float32(0))
        hi = np.nextafter(r, np.float32(np.inf))
        fx = Fraction(float(x))
        mid_lo = (Fraction(float(lo)) + Fraction(float(r))) / 2
        mid_hi = (Fraction(float(r)) + Fraction(float(hi))) / 2
        assert mid_lo * mid_lo <= fx <= mid_hi * mid_hi


def test_sqrt_closed_forms():
    k = np.arange(0, 101, dtype=np.float32)
    assert np.array_equal(ops.sqrt(k * k), k)                  # sqrt(k^2) = k
    assert ops.sqrt(np.float32(2.0)) == np.float32(1.41421356)
    assert ops.sqrt(np.float16(4.0), np.float16) == np.float16(2.0)


def test_sqrt_of_binary32_to_binary16_rounds_through_binary32():
    # 469.33163 as binary32 is 469.331634521484375 = 2^-15 * 15379059.  Its
    # root lies just above 21.6640625: 21.6640625^2 = 469.33160400390625,
    # and 21.6640625 + 2^-20 (half a binary32 ulp at 16..32) squares to
    # 21.6640625^2 + 2 * 21.6640625 * 2^-20 + 2^-40 > 469.3316731 > x.  So
    # the binary32 root is 21.6640625 exactly, halfway between the binary16
    # neighbours 21.65625 (significand 0x56A, even) and 21.671875 (0x56B):
    # the binary16 result is the even one, 21.65625, while one rounding of
    # the exact root would give 21.671875.
    x = np.float32(469.33163)
    assert Fraction(float(x)) == Fraction(15379059, 2 ** 15)
    assert Fraction(21.6640625) ** 2 < Fraction(float(x)) < (Fraction(21.6640625) + Fraction(1, 2 ** 20)) ** 2
    assert ops.sqrt(x, np.float32) == np.float32(21.6640625)
    assert ops.sqrt(x, np.float16) == np.float16(21.65625)
    assert int(np.float16(21.65625).view(np.uint16)) & 0x3FF == 0x16A          # even significand
    # binary16 inputs: the two roundings equal one (24 >= 2 * 11 + 2)
    h = np.arange(0x3C00, 0x7C00, 7, dtype=np.uint16).view(np.float16)
    exact = np.sqrt(h.astype(np.float64)).astype(np.float16)
    assert np.array_equal(ops.sqrt(h, np.float16).view(np.uint16), exact.view(np.uint16))


def test_exp_against_high_precision():
    mpmath.mp.prec = 200
    xs = np.float16(np.linspace(-4, 4, 4001)).astype(np.float32)
    got = ops.exp(xs, np.float32)
    ulp_err = []
    for x, g in zip(xs, got):
        man, ex = mpmath.exp(mpmath.mpf(float(x))).man_exp  # binary mantissa/exponent, ~200 bits
        q = Fraction(int(man)) * (Fraction(2) ** int(ex))
        want = round_exact(q, np.float32)
        ulp_err.append(abs(int(np.float32(g).view(np.int32)) - int(np.float32(want).view(np.int32))))
    # the oracle is the correctly-rounded value or 1 ulp from it, and almost always exact
    assert max(ulp_err) <= 1
    assert sum(ulp_err) <= 2


def test_exp_closed_forms():
    assert ops.exp(np.float32(0.0)) == np.float32(1.0)
    assert ops.exp(np.float32(-0.0)) == np.float32(1.0)
    assert ops.exp(np.float32(1.0)) == np.float32(math.e)
    assert ops.exp(np.float32(-np.inf)) == np.float32(0.0)


def test_zero_is_positive_zero():
    z = ops.zero((4, 4), np.float32)
    assert not np.any(z.view(np.uint32))
