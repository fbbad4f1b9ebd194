"""Pins of the oracle's store with reduce-add: brute force over tiny tensors,
modular uint32 wrap-around, and the single-contribution case equal to the
plain IEEE addition."""
import itertools

import numpy as np
import pytest

from oracle import ops
from oracle import reference as REF


def _brute(dst, src):
    out = dst.astype(object).copy()
    for i in itertools.product(*[range(n) for n in src.shape]):
        j = tuple(0 if m == 1 else k for k, m in zip(i, dst.shape))
        out[j] = out[j] + int(src[i]) if dst.dtype == np.uint32 else out[j] + float(src[i])
    return out


def test_reduce_bruteforce_uint32_wraps():
    rng = np.random.default_rng(3)
    src = rng.integers(0, 2**32, size=(5, 3, 4), dtype=np.uint64).astype(np.uint32)
    dst = rng.integers(0, 2**32, size=(1, 3, 4), dtype=np.uint64).astype(np.uint32)
    got = REF.tile_reduce_add(dst, src)
    want = np.vectorize(lambda v: v % 2**32)(_brute(dst, src)).astype(np.uint32)
    assert np.array_equal(got, want)
    # a sum that wraps: 2**31 + 2**31 + 5 -> 5
    assert REF.tile_reduce_add(np.array([[5]], np.uint32), np.array([[2**31], [2**31]], np.uint32))[0, 0] == 5


@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_reduce_bruteforce_exact_float_sums(dt):
    # small integers: every partial sum is exact, so any order gives this
    rng = np.random.default_rng(4)
    src = rng.integers(-8, 9, size=(6, 2, 7)).astype(dt)
    dst = rng.integers(-8, 9, size=(1, 2, 7)).astype(dt)
    got = REF.tile_reduce_add(dst, src)
    want = np.array(_brute(dst, src), dtype=np.float64).astype(dt)
    assert np.array_equal(got, want)
    # two reduced dims at once
    src2 = rng.integers(-8, 9, size=(3, 4, 5)).astype(dt)
    dst2 = np.zeros((1, 1, 5), dt)
    assert np.array_equal(REF.tile_reduce_add(dst2, src2), src2.astype(np.float64).sum(axis=(0, 1), keepdims=True).astype(dt))


def test_reduce_single_contribution_is_ieee_add():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((4, 64)).astype(np.float32)
    y = rng.standard_normal((4, 64)).astype(np.float32)
    assert np.array_equal(REF.tile_reduce_add(y, x).view(np.uint32), ops.add(y, x, np.float32).view(np.uint32))
    # and the float32 sum of two float32 numbers rounded once (numpy's own add)
    assert np.array_equal(REF.tile_reduce_add(y, x).view(np.uint32), (y + x).view(np.uint32))


def test_reduce_rejects_bad_shapes():
    with pytest.raises(ValueError):
        REF.tile_reduce_add(np.zeros((2, 3), np.float32), np.zeros((4, 3), np.float32))
    with pytest.raises(ValueError):
        REF.tile_reduce_add(np.zeros((3,), np.float32), np.zeros((4, 3), np.float32))


def test_reduce_rows_exact_then_rounded_once():
    from fractions import Fraction
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((7, 33)) * 10.0 ** rng.integers(-6, 7, (7, 33))).astype(np.float32)
    got = REF.reduce_rows(x)
    for r in range(7):
        exact = sum(Fraction(float(v)) for v in x[r])
        # float32(exact) by round-to-nearest: compare against both neighbours
        f = np.float32(float(exact))
        assert got[r] == f
        lo, hi = np.nextafter(f, np.float32(-np.inf)), np.nextafter(f, np.float32(np.inf))
        assert abs(Fraction(float(f)) - exact) <= abs(Fraction(float(lo)) - exact)
        assert abs(Fraction(float(f)) - exact) <= abs(Fraction(float(hi)) - exact)


def test_reduce_rows_closed_forms():
    n = 1000
    x = np.arange(1, n + 1, dtype=np.float32)[None, :]
    assert REF.reduce_rows(x)[0] == n * (n + 1) // 2
    # cancellation: plain float32 left-to-right loses the 1, the exact sum keeps it
    y = np.array([[1e8, 1.0, -1e8]], np.float32)
    assert REF.reduce_rows(y)[0] == 1.0
    assert REF.reduce_rows(np.zeros((3, 0), np.float32)).tolist() == [0.0, 0.0, 0.0]
    h = np.full((2, 2048), 0.5, np.float16)
    assert REF.reduce_rows(h).tolist() == [1024.0, 1024.0]


def test_recursive_sum_bound_holds_for_left_to_right_sums():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((50, 1024)).astype(np.float32)
    ltr = np.zeros(50, np.float32)
    for c in range(1024):
        ltr = ltr + x[:, c]                       # binary32 left to right
    err = np.abs(ltr.astype(np.float64) - REF.reduce_rows(x).astype(np.float64))
    ulp = np.spacing(np.abs(REF.reduce_rows(x)))
    assert np.all(err <= REF.recursive_sum_bound(x, 1023) + ulp)
