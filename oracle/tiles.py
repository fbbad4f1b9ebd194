"""LDS byte image of a tile and the tiled data path built on it (oracle).

Sources
-------
* "copy_async -> tma", "Demonstration program": the tile goes global ->
  shared (swizzled layout) and is read back with a plain CTA copy; the
  descriptor's last encode argument is the out-of-bounds fill (0).
* "copy_async -> ldgsts", "Demonstration program" and "Algorithm" step 2: the
  same transfer as per-thread asynchronous vector copies, then a CTA copy out.
* "elementwise -> smem", "Demonstration program": copy in, apply the op on the
  shared tile, copy out.

The image of tile ``t`` is built element by element: enumerate the image
axes row-major, compute each element's tensor coordinates, read it (or zero
when out of bounds: the out-of-bounds fill value of the descriptor is 0) and
place its bytes at the swizzled LDS offset.  Scattering reverses it and
skips out-of-bounds elements.  Pure Python loops: meant for tiles of a few
KiB.
"""
from __future__ import annotations

import numpy as np

from . import plan as _plan


def _element_offset(coords, strides) -> int:
    return sum(int(c) * int(s) for c, s in zip(coords, strides))


def lds_image(storage: np.ndarray, p: _plan.Plan, tile_index: int) -> bytes:
    """Raw LDS bytes of tile ``tile_index`` of the tensor in ``storage``.

    ``storage`` is the flat element buffer the descriptor's strides index.
    """
    raw = storage.view(np.uint8)
    es = p.esize
    origin = _plan.tile_origin(p.shape, p.box, tile_index)
    image = bytearray(p.tile_bytes)
    for e, rel in enumerate(image_coords_cached(p)):
        coords = [o + r for o, r in zip(origin, rel)]
        dst = _plan.lds_offset(p, e * es)
        if all(c < n for c, n in zip(coords, p.shape)):
            src = _element_offset(coords, p.strides) * es
            image[dst:dst + es] = raw[src:src + es].tobytes()
        else:
            image[dst:dst + es] = bytes(es)
    return bytes(image)


def scatter_image(image: bytes, out_storage: np.ndarray, out_strides, p: _plan.Plan,
                  tile_index: int, out_esize: int | None = None) -> None:
    """Write an LDS image back to a tensor (OOB elements are dropped).

    ``out_esize`` lets the image hold a wider element than ``p`` (an op whose
    output type differs); the image is then read with the output element size.
    """
    raw = out_storage.view(np.uint8)
    es = out_esize or p.esize
    origin = _plan.tile_origin(p.shape, p.box, tile_index)
    for e, rel in enumerate(image_coords_cached(p)):
        coords = [o + r for o, r in zip(origin, rel)]
        if not all(c < n for c, n in zip(coords, p.shape)):
            continue
        src = _plan.lds_offset(p, e * es)
        dst = _element_offset(coords, out_strides) * es
        raw[dst:dst + es] = np.frombuffer(image[src:src + es], dtype=np.uint8)


_coord_cache: dict = {}


def image_coords_cached(p: _plan.Plan):
    key = tuple((a.count, a.dim, a.step) for a in p.image_axes) + (len(p.shape),)
    if key not in _coord_cache:
        _coord_cache[key] = _plan.image_coords(p)
    return _coord_cache[key]


def image_elements(image: bytes, p: _plan.Plan, dtype) -> np.ndarray:
    """Elements of an image in logical (unswizzled) order."""
    dt = np.dtype(dtype)
    es = dt.itemsize
    n = len(image) // es
    out = bytearray(len(image))
    for e in range(n):
        src = _plan.lds_offset(p, e * es)
        out[e * es:(e + 1) * es] = image[src:src + es]
    return np.frombuffer(bytes(out), dtype=dt)


def elements_to_image(values: np.ndarray, p: _plan.Plan) -> bytes:
    """Inverse of ``image_elements``: place logical-order elements swizzled."""
    es = values.dtype.itemsize
    src = values.tobytes()
    out = bytearray(len(src))
    for e in range(len(values)):
        dst = _plan.lds_offset(p, e * es)
        out[dst:dst + es] = src[e * es:(e + 1) * es]
    return bytes(out)


def tiled_copy(storage: np.ndarray, p: _plan.Plan, out_storage: np.ndarray, out_strides) -> None:
    """Copy every tile global -> LDS image -> global."""
    n_tiles = int(np.prod(_plan.tile_grid(p.shape, p.box)))
    for t in range(n_tiles):
        scatter_image(lds_image(storage, p, t), out_storage, out_strides, p, t)


def tiled_ewise(fn, in_storages, p: _plan.Plan, in_dtype, out_storage: np.ndarray,
                out_strides, out_dtype) -> None:
    """Apply ``fn`` (elementwise over equal-shape arrays) tile by tile through
    the LDS images of every input; the result is staged as an image of the
    output type and scattered."""
    n_tiles = int(np.prod(_plan.tile_grid(p.shape, p.box)))
    for t in range(n_tiles):
        ins = [image_elements(lds_image(s, p, t), p, in_dtype) for s in in_storages]
        res = np.asarray(fn(*ins)).astype(out_dtype)
        scatter_image(elements_to_image(res, p), out_storage, out_strides, p, t,
                      out_esize=np.dtype(out_dtype).itemsize)
