"""Seeded synthetic inputs for the five tile-pipelining workloads.

This module only draws random numbers and lays them out in host buffers
(shape, dtype, value distribution, row pitch).  It holds none of the
arithmetic of the method: no tiling, no swizzle, no elementwise op.  Both
the CPU oracle and the HIP path consume exactly these arrays.

Seeds default to the workload number (1..5); every draw goes through
``numpy.random.default_rng(seed)``.

Workloads (sizes are parameters so tests can shrink them):

1. one 8x256 float16 tile; values are uniform random 16-bit patterns with
   the NaN/Inf exponent (0x1F) excluded;
2. a batch of 32x32 float32 tiles, values uniform in [0, 1e4);
3. a [128, 500, 1024] float16 tensor, N(0, 1) rounded to float16;
4. a [128, 500, 1024] float32 tensor x ~ N(0, 1) with per-row scalars
   a, b ~ U(-2, 2) of shape [128, 500];
5. a (4, 8, 64, 128, 256) float16 tensor x ~ U(-4, 4) stored with a row
   pitch of 264 elements; the 8 pad elements per row hold a float16 NaN
   sentinel so that any read of them is visible downstream.
"""
from __future__ import annotations

import numpy as np

F16_PAD_SENTINEL = np.uint16(0x7E5A)  # a quiet float16 NaN with a recognisable payload


def tile_bits_f16(shape=(8, 256), seed: int = 1) -> np.ndarray:
    """Uniform float16 bit patterns over all finite encodings (exponent != 0x1F)."""
    rng = np.random.default_rng(seed)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    filled = 0
    while filled < n:
        cand = rng.integers(0, 1 << 16, size=2 * (n - filled), dtype=np.uint32).astype(np.uint16)
        cand = cand[((cand >> 10) & 0x1F) != 0x1F]
        take = min(len(cand), n - filled)
        out[filled:filled + take] = cand[:take]
        filled += take
    return out.reshape(shape).view(np.float16)


def sqrt_tiles_f32(tiles: int = 65536, tile=(32, 32), seed: int = 2) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.random((tiles,) + tuple(tile), dtype=np.float32) * np.float32(1e4)).astype(np.float32)


def normal_f16(shape=(128, 500, 1024), seed: int = 3) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.standard_normal(shape, dtype=np.float32).astype(np.float16)


def fma_rows_f32(shape=(128, 500, 1024), seed: int = 4):
    """x ~ N(0,1) of ``shape``; a, b ~ U(-2, 2) of ``shape[:-1]`` (one scalar per row)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape, dtype=np.float32)
    a = rng.uniform(-2.0, 2.0, size=shape[:-1]).astype(np.float32)
    b = rng.uniform(-2.0, 2.0, size=shape[:-1]).astype(np.float32)
    return x, a, b


def padded_uniform_f16(shape=(4, 8, 64, 128, 256), pitch: int = 264, seed: int = 5, lo=-4.0, hi=4.0):
    """x ~ U(lo, hi) in float16, stored with innermost-row pitch ``pitch``.

    Returns ``(storage, strides)``: ``storage`` is the flat float16 buffer
    (pad elements hold ``F16_PAD_SENTINEL``), ``strides`` are element strides
    outermost-first with the innermost stride 1 and the row stride ``pitch``.
    """
    shape = tuple(int(s) for s in shape)
    assert pitch >= shape[-1]
    rng = np.random.default_rng(seed)
    vals = rng.uniform(lo, hi, size=shape).astype(np.float16)
    strides = [1, pitch]
    for ext in reversed(shape[1:-1]):
        strides.append(strides[-1] * ext)
    strides = tuple(reversed(strides))
    rows = int(np.prod(shape[:-1]))
    storage = np.full(rows * pitch, F16_PAD_SENTINEL, dtype=np.uint16).view(np.float16)
    view = np.lib.stride_tricks.as_strided(
        storage, shape=shape, strides=tuple(s * 2 for s in strides))
    view[...] = vals
    return storage, strides


def strided_view(storage: np.ndarray, shape, strides) -> np.ndarray:
    """Read-only numpy view of ``storage`` with element ``strides``."""
    item = storage.dtype.itemsize
    return np.lib.stride_tricks.as_strided(
        storage, shape=tuple(shape), strides=tuple(int(s) * item for s in strides), writeable=False)
