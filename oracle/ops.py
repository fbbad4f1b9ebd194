"""Elementwise ops with IEEE-754 round-to-nearest-even results (oracle).

Source: "elementwise -> smem", "What it accepts" (op registry: unary sqrt /
exp / zero, binary add / mul, fma), "Generated CUDA" (the fp32 tile's sqrt is
taken per component) and "How inputs change the algorithm" (fma is
a * b + c).

Precision readings:
* add and mul compute in binary64 from exactly widened inputs (all of one
  type) and round once to that type.  The extra rounding through binary64 is
  harmless because 53 >= 2p + 2 for p = 24 and p = 11 (double rounding is
  innocuous for these operations).
* fma is fused: ONE rounding of the exact a * x + b.  The product of two
  binary32 (or binary16) values is exact in binary64; the sum is formed in
  binary64 with round-to-odd (TwoSum error term, then force the last bit odd
  when inexact) and rounded once to the output type.  Round-to-odd at
  53 >= p + 2 bits makes the second rounding correct (Boldo & Melquiond,
  "Emulation of FMA and correctly rounded sums: proved algorithms using
  rounding to odd", IEEE TC 2008).
* sqrt and exp compute in binary32 (the unary ops of "elementwise -> smem"
  take float16 or float32 and compute in float32; reading adopted): the
  result is the binary32 one (sqrt correctly rounded, exp(x) in binary64
  rounded) converted to the output type.  With binary32 or binary16 inputs
  and a binary32 output that is one rounding.  A binary16 output of a
  binary32 input rounds twice: a binary32 result that falls exactly halfway
  between two binary16 values resolves to the even one, whatever side the
  exact value lay on.  (For binary16 inputs and output the two roundings
  equal one: 24 >= 2 * 11 + 2.)
* exp(x) in binary64 lies within half an ulp plus 2^-53 relative of the
  exact value; a result within 1 ulp of the oracle's is accepted for exp.
* zero writes +0 (all bits clear).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x).astype(np.float64)


def sqrt(x, out_dtype=np.float32) -> np.ndarray:
    return np.sqrt(_f64(x)).astype(np.float32).astype(out_dtype)


def exp(x, out_dtype=np.float32) -> np.ndarray:
    with np.errstate(over="ignore"):
        return np.exp(_f64(x)).astype(np.float32).astype(out_dtype)


def add(a, b, out_dtype=np.float32) -> np.ndarray:
    return (_f64(a) + _f64(b)).astype(out_dtype)


def mul(a, b, out_dtype=np.float32) -> np.ndarray:
    return (_f64(a) * _f64(b)).astype(out_dtype)


def zero(shape, out_dtype=np.float32) -> np.ndarray:
    return np.zeros(shape, dtype=out_dtype)


def _sum_round_to_odd(p: np.ndarray, c: np.ndarray) -> np.ndarray:
    """p + c in binary64 rounded to odd (p, c finite binary64)."""
    s = p + c
    # TwoSum (Knuth): err is exactly (p + c) - s.
    bv = s - p
    av = s - bv
    err = (p - av) + (c - bv)
    bits = s.view(np.int64)
    need = (err != 0) & ((bits & 1) == 0)
    toward = np.where(err > 0, np.inf, -np.inf)
    return np.where(need, np.nextafter(s, toward), s)


def fma(a, x, b, out_dtype=np.float32) -> np.ndarray:
    """Correctly rounded a * x + b (single rounding)."""
    a64, x64, b64 = np.broadcast_arrays(_f64(a), _f64(x), _f64(b))
    with np.errstate(invalid="ignore", over="ignore"):
        prod = a64 * x64                      # exact for binary32 / binary16 inputs
        finite = np.isfinite(prod) & np.isfinite(b64)
        safe_p = np.where(finite, prod, 0.0)
        safe_b = np.where(finite, b64, 0.0)
        ro = _sum_round_to_odd(safe_p, safe_b)
        plain = prod + b64                    # infinities / NaN propagate as IEEE
        return np.where(finite, ro, plain).astype(out_dtype)


UNARY = {"sqrt": sqrt, "exp": exp}
BINARY = {"add": add, "mul": mul}
