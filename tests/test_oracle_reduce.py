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


def _round_exact(q, dt):
    """Rational q rounded to nearest in numpy float type dt, ties to even,
    decided by exact rational distances (no intermediate binary64 rounding
    can decide it: the binary64 guess only picks the three candidates)."""
    from fractions import Fraction
    f = dt(float(q))
    cands = [np.nextafter(f, dt(-np.inf)), f, np.nextafter(f, dt(np.inf))]
    cands = [c for c in cands if np.isfinite(c)]
    best = min(abs(Fraction(float(c)) - q) for c in cands)
    ties = [c for c in cands if abs(Fraction(float(c)) - q) == best]
    if len(ties) == 1:
        return ties[0]
    bits = np.dtype(dt).type
    ui = np.uint16 if dt == np.float16 else np.uint32
    return [c for c in ties if int(np.array(c, dt).view(ui)) % 2 == 0][0]


def _exact_sum(values):
    from fractions import Fraction
    return sum((Fraction(float(v)) for v in values), Fraction(0))


def test_reduce_rows_exact_then_rounded_once():
    rng = np.random.default_rng(6)
    x = (rng.standard_normal((7, 33)) * 10.0 ** rng.integers(-6, 7, (7, 33))).astype(np.float32)
    got = REF.reduce_rows(x)
    for r in range(7):
        assert got[r] == _round_exact(_exact_sum(x[r]), np.float32)


def test_reduce_rows_single_rounding_at_a_binary64_sticky_bit():
    # 1 + 2**-24 is the binary32 midpoint between 1 and 1 + 2**-23; the
    # 2**-80 term puts the exact sum just above it, so it rounds up.  Summing
    # into binary64 first drops the 2**-80 (half an ulp of binary64 is
    # 2**-53) and the tie then goes to the even neighbour, 1.
    x = np.array([[1.0, 2.0 ** -24, 2.0 ** -80]], np.float32)
    assert REF.reduce_rows(x)[0] == np.float32(1 + 2.0 ** -23)
    # the same below the midpoint
    x = np.array([[1.0, 2.0 ** -24, -(2.0 ** -80)]], np.float32)
    assert REF.reduce_rows(x)[0] == np.float32(1.0)
    # and for negative sums (truncation toward zero mirrors)
    x = np.array([[-1.0, -(2.0 ** -24), -(2.0 ** -80)]], np.float32)
    assert REF.reduce_rows(x)[0] == np.float32(-(1 + 2.0 ** -23))
    # an exact tie stays a tie: ties to even
    x = np.array([[1.0, 2.0 ** -24]], np.float32)
    assert REF.reduce_rows(x)[0] == np.float32(1.0)
    x = np.array([[1.0 + 2.0 ** -23, 2.0 ** -24]], np.float32)
    assert REF.reduce_rows(x)[0] == np.float32(1.0 + 2.0 ** -22)


def test_reduce_rows_random_near_ties_against_exact_rounding():
    # rows built around binary32 midpoints with tiny residues far below the
    # binary64 precision of the sum: every one needs the single rounding
    rng = np.random.default_rng(11)
    rows = []
    for _ in range(300):
        big = np.float32(rng.uniform(1, 2)) * np.float32(2.0 ** int(rng.integers(-4, 5)))
        half_ulp = np.spacing(big) / 2
        tail = float(rng.choice([-1, 1])) * 2.0 ** -int(rng.integers(60, 120))
        extra = [float(v) for v in rng.standard_normal(int(rng.integers(0, 4))).astype(np.float32) * 2.0 ** -40]
        rows.append([float(big), float(half_ulp), tail] + extra + [0.0] * (6 - 3 - len(extra)))
    x = np.array(rows, dtype=np.float32)
    got = REF.reduce_rows(x)
    for r in range(len(rows)):
        assert got[r] == _round_exact(_exact_sum(x[r]), np.float32), x[r]


def test_reduce_add_float_single_rounding():
    # store with reduce-add into float32: dst 1, contributions 2**-24 and
    # 2**-80: the exact sum lies just above the binary32 midpoint
    dst = np.array([[1.0]], np.float32)
    src = np.array([[2.0 ** -24], [2.0 ** -80]], np.float32)
    assert REF.tile_reduce_add(dst, src)[0, 0] == np.float32(1 + 2.0 ** -23)
    # float16: 1 + 2**-11 is the binary16 midpoint between 1 and 1 + 2**-10;
    # the subnormal 2**-24 puts the exact sum above it.  Rounding the partial
    # sum 1 + 2**-11 to binary16 first would give 1 (ties to even), and 1 +
    # 2**-24 rounds to 1 again.
    dst16 = np.zeros((1, 1), np.float16)
    src16 = np.array([[1.0], [2.0 ** -11], [2.0 ** -24]], np.float16)
    assert REF.tile_reduce_add(dst16, src16)[0, 0] == np.float16(1 + 2.0 ** -10)
    h = np.float16(1.0)
    for v in src16[1:, 0]:
        h = np.float16(h + v)
    assert h == np.float16(1.0)


@pytest.mark.parametrize("dt", [np.float32, np.float16])
def test_reduce_add_random_against_exact_rounding(dt):
    rng = np.random.default_rng(12)
    src = (rng.standard_normal((9, 3, 5)) * 2.0 ** rng.integers(-12, 12, (9, 3, 5))).astype(dt)
    dst = rng.standard_normal((1, 3, 5)).astype(dt)
    got = REF.tile_reduce_add(dst, src)
    for j in range(3):
        for k in range(5):
            want = _round_exact(_exact_sum(list(src[:, j, k]) + [dst[0, j, k]]), dt)
            assert got[0, j, k] == want


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
