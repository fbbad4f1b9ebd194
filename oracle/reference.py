"""Plain definitions every tiled / pipelined result must equal (oracle).

* tile copy (global -> LDS -> global): the output equals the input bit for
  bit; tiling, swizzle, the stage ring and the out-of-bounds fill never reach
  the output ("copy_async -> tma" and "copy_async -> ldgsts", "Demonstration
  program": the tile is read back unchanged).
* elementwise: y[i] = op(inputs[i]) element by element ("elementwise ->
  smem", "Demonstration program": the tile equals sqrt(A)).
* streamed elementwise with per-row scalars: for a tensor x whose rows are
  its innermost runs, y[r, c] = op(a[r], x[r, c], b[r]) with
  fma = a*x + b, add = x + b, mul = a*x; unary ops ignore a and b.
* store with reduce-add ("copy_async -> tma", "How inputs change the
  algorithm": a shared -> global copy with a reduce op, e.g. add): every
  staged element is added into the destination element it maps to.  With
  a destination of extent 1 along some dims, every source element along
  those dims adds into the same destination element:
  dst'[j] = dst[j] + sum of src[i] over the i that map to j.  Integers wrap
  modulo 2**32.  For floats the page fixes no order of the additions;
  reading adopted: the sum is the exact one rounded once to the
  destination type, which every order of IEEE additions reproduces when
  each partial sum is exactly representable (and always with a single
  contribution).
* row reduction ("Add TMA support for circular buffering pass", "Testing
  Setup": the Reduction and InnerPersistent schedules over circular-
  buffered loads): y[row] = sum of x[row, c] over the innermost dim, the
  exact sum rounded once to binary32.  Reading adopted: the page names the
  schedule, not an accumulation order; the exact sum is the one definition
  every order approximates (the GPU's fixed order is compared against it
  within the textbook bound for recursive summation).
"""
from __future__ import annotations

import itertools
import math
import struct

import numpy as np

from . import ops


def _odd_neighbour(t: float, away: float) -> float:
    """Of t and its binary64 neighbour in the direction ``away`` (away from
    zero), the one whose significand is odd."""
    bits = struct.unpack("<q", struct.pack("<d", t))[0]
    return t if bits & 1 else math.nextafter(t, away)


def _sum_to_odd(values) -> float:
    """The exact sum of finite binary64 ``values`` rounded to binary64 with
    round-to-odd: truncated toward zero to 53 bits, and when that dropped
    anything, the odd one of the two neighbours enclosing the exact sum.
    A binary64 round-to-odd result rounded to nearest into a format of at most
    51 significand bits gives the exact value rounded once to nearest in that
    format (Boldo and Melquiond, "Emulation of FMA and correctly rounded sums:
    proved algorithms using rounding to odd", IEEE Trans. Computers 2008).

    ``math.fsum`` gives s, the exact sum rounded to nearest binary64; a second
    ``fsum`` of the values and -s gives the sign of the exact residual
    (exact - s), which is a nonzero multiple of 2**-1074 whenever the sum
    was inexact, so it never rounds to zero."""
    vals = values if isinstance(values, list) else list(values)
    s = math.fsum(vals)
    if not math.isfinite(s) or s == 0.0:
        return s
    r = math.fsum(itertools.chain(vals, (-s,)))
    if r == 0.0:
        return s
    away = math.inf if s > 0 else -math.inf
    # truncation toward zero: s itself when the exact sum lies beyond it
    # (further from zero), else the neighbour of s toward zero
    t = s if (r > 0) == (s > 0) else math.nextafter(s, 0.0)
    return _odd_neighbour(t, away)


def sum_rounded_once(rows: np.ndarray, out_dtype) -> np.ndarray:
    """Exact sum of each row of ``rows`` (a 2-D array of binary16/32/64
    values), rounded once to nearest-even in ``out_dtype`` (binary16 or
    binary32)."""
    rows = np.asarray(rows, dtype=np.float64)
    ro = np.array([_sum_to_odd(r) for r in rows.tolist()], dtype=np.float64)
    with np.errstate(over="ignore"):
        return ro.astype(out_dtype)


def tile_copy(x: np.ndarray) -> np.ndarray:
    return np.array(x, copy=True)


def ewise(op: str, inputs, out_dtype) -> np.ndarray:
    """Elementwise op over equal-shape inputs (fma takes a, b, c -> a*b + c)."""
    if op == "zero":
        return ops.zero(np.shape(inputs[0]) if inputs else (), out_dtype)
    if op in ops.UNARY:
        return ops.UNARY[op](inputs[0], out_dtype)
    if op in ops.BINARY:
        return ops.BINARY[op](inputs[0], inputs[1], out_dtype)
    if op == "fma":
        return ops.fma(inputs[0], inputs[1], inputs[2], out_dtype)
    raise ValueError(f"unknown op {op}")


def stream_ewise(op: str, x: np.ndarray, a=None, b=None, out_dtype=np.float32) -> np.ndarray:
    """y = op(a[row], x, b[row]) with one scalar of a and b per innermost row."""
    if op in ("zero", "sqrt", "exp"):
        return ewise(op, [x], out_dtype)
    a_b = None if a is None else np.asarray(a)[..., None]
    b_b = None if b is None else np.asarray(b)[..., None]
    if op == "fma":
        return ops.fma(a_b, x, b_b, out_dtype)
    if op == "add":
        return ops.add(x, b_b, out_dtype)
    if op == "mul":
        return ops.mul(a_b, x, out_dtype)
    raise ValueError(f"unknown op {op}")


def tile_reduce_add(dst: np.ndarray, src: np.ndarray) -> np.ndarray:
    """dst + src summed over the dims where dst has extent 1 and src more."""
    dst = np.asarray(dst)
    src = np.asarray(src)
    if dst.ndim != src.ndim:
        raise ValueError("dst and src must have the same rank")
    axes = []
    for d, (m, n) in enumerate(zip(dst.shape, src.shape)):
        if m == n:
            continue
        if m != 1:
            raise ValueError("dst extents must equal src's or be 1")
        axes.append(d)
    if dst.dtype == np.uint32:
        total = src.astype(np.uint64).sum(axis=tuple(axes), keepdims=True) + dst.astype(np.uint64)
        return (total % (1 << 32)).astype(np.uint32)
    if dst.dtype in (np.float16, np.float32):
        # contributions to each destination element: the summed dims moved
        # last, then the destination's own value
        kept = [d for d in range(src.ndim) if d not in axes]
        contrib = np.transpose(src, kept + axes).reshape(dst.size, -1).astype(np.float64)
        rows = np.concatenate([contrib, dst.reshape(dst.size, 1).astype(np.float64)], axis=1)
        return sum_rounded_once(rows, dst.dtype).reshape(dst.shape)
    raise ValueError("reduce-add takes uint32, float16 or float32")


def reduce_rows(x: np.ndarray) -> np.ndarray:
    """Exact sum of every innermost row, rounded once to float32."""
    x = np.asarray(x)
    n_rows = int(np.prod(x.shape[:-1]))
    rows = x.reshape(n_rows, x.shape[-1]).astype(np.float64)
    return sum_rounded_once(rows, np.float32).reshape(x.shape[:-1])


def recursive_sum_bound(x: np.ndarray, n_adds: int) -> np.ndarray:
    """Per-row bound on |computed - exact| for any order of n_adds binary32
    additions of the row's values: gamma_n * sum |x|, gamma_n = n u / (1 - n u),
    u = 2**-24 (recursive summation, Higham, Accuracy and Stability of
    Numerical Algorithms, section 4.2)."""
    u = 2.0 ** -24
    g = n_adds * u / (1 - n_adds * u)
    return g * np.abs(np.asarray(x, dtype=np.float64)).sum(axis=-1)
