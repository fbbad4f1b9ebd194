"""Pins of the oracle's LDS images and tiled data path: hand-worked image
bytes, copy identity, zero fill out of bounds, and the tiled ops equal to
the plain elementwise definitions."""
import numpy as np

import workloads as W
from oracle import plan as P
from oracle import reference as REF
from oracle import tiles as T


def test_c1_image_hand_values():
    # 8x256 float16 with element value = its index (as uint16 bits).
    x = np.arange(8 * 256, dtype=np.uint16)
    p = P.plan("f16", (8, 256), (256, 1), (8, 256), P.SWIZZLE_128B, threads=64)
    img = np.frombuffer(T.lds_image(x, p, 0), dtype=np.uint16)
    # image = 4 atoms of 1 KiB (atom a holds columns 64a..64a+63 of all 8 rows);
    # inside an atom, row r's logical 16-byte chunk c sits in physical chunk c ^ r.
    def at(atom, row, phys_chunk, k):
        return int(img[(atom * 1024 + row * 128 + phys_chunk * 16) // 2 + k])
    assert at(0, 0, 0, 0) == 0                       # row 0 is unswizzled
    assert at(0, 1, 1, 0) == 256 + 0                 # row 1, logical chunk 0 -> physical 1
    assert at(0, 1, 0, 0) == 256 + 8                 # row 1, logical chunk 1 -> physical 0
    assert at(2, 3, 6, 5) == 3 * 256 + 128 + 5 * 8 + 5   # atom 2, row 3, logical chunk 5
    assert at(3, 7, 0, 7) == 7 * 256 + 192 + 7 * 8 + 7   # atom 3, row 7, logical chunk 7


def test_c1_copy_identity_through_image():
    x = W.tile_bits_f16((8, 256), seed=1)
    assert not np.any(((x.view(np.uint16) >> 10) & 0x1F) == 0x1F)     # no NaN/Inf drawn
    p = P.plan("f16", (8, 256), (256, 1), (8, 256), P.SWIZZLE_128B, threads=64)
    img = T.lds_image(x.reshape(-1), p, 0)
    assert img != x.tobytes()                                          # the swizzle moved bytes
    out = np.zeros(8 * 256, np.float16)
    T.tiled_copy(x.reshape(-1), p, out, (256, 1))
    assert np.array_equal(out.view(np.uint16), x.reshape(-1).view(np.uint16))


def test_ragged_tiles_zero_fill_and_identity():
    # a small version of the [128, 500, 1024] workload: tails in rows and columns
    shape, box = (2, 20, 64), (1, 8, 32)
    x = W.normal_f16(shape, seed=3)
    p = P.plan("f16", shape, (20 * 64, 64, 1), box, threads=128)
    # tile (0, 2, 1) covers rows 16..23 of which 16..19 exist
    t = np.ravel_multi_index((0, 2, 1), P.tile_grid(shape, box))
    img = np.frombuffer(T.lds_image(x.reshape(-1), p, t), dtype=np.float16).reshape(8, 32)
    assert np.array_equal(img[:4], x[0, 16:20, 32:64])
    assert not np.any(img[4:].view(np.uint16))                         # out-of-bounds rows are +0
    out = np.zeros(x.size, np.float16)
    T.tiled_copy(x.reshape(-1), p, out, (20 * 64, 64, 1))
    assert np.array_equal(out.reshape(shape).view(np.uint16), REF.tile_copy(x).view(np.uint16))


def test_tiled_sqrt_equals_plain_definition():
    x = W.sqrt_tiles_f32(tiles=6, seed=2)
    p = P.plan("f32", x.shape, (1024, 32, 1), (1, 32, 32), threads=256, copy_only=False)
    assert (p.vec, p.outer) == (4, 1)
    out = np.zeros(x.size, np.float32)
    T.tiled_ewise(lambda v: REF.ewise("sqrt", [v], np.float32), [x.reshape(-1)], p, np.float32,
                  out, (1024, 32, 1), np.float32)
    assert np.array_equal(out.reshape(x.shape), REF.ewise("sqrt", [x], np.float32))


def test_padded_rank5_exp_never_reads_pad():
    shape, pitch = (1, 2, 2, 8, 64), 72
    storage, strides = W.padded_uniform_f16(shape, pitch=pitch, seed=5)
    p = P.plan("f16", shape, strides, (1, 1, 1, 8, 64), P.SWIZZLE_128B, threads=64, copy_only=False)
    # dim 2 (box 1) merges with the fully boxed 8-row dim 3 (contiguous: 576 = 8 * 72);
    # the pitch keeps dims 3 and 4 apart; dim 0 (extent 1) is dropped.
    assert p.rank == 3 and p.encode_args()[1] == [64, 16, 2]
    out = np.full(int(np.prod(shape)), np.nan, np.float32)
    packed = tuple(int(np.prod(shape[k + 1:])) for k in range(len(shape)))
    T.tiled_ewise(lambda v: REF.ewise("exp", [v], np.float32), [storage], p, np.float16,
                  out, packed, np.float32)
    x = W.strided_view(storage, shape, strides)
    assert np.array_equal(out.reshape(shape), REF.ewise("exp", [x], np.float32))
    assert not np.any(np.isnan(out))


def test_stream_fma_reference_rows():
    x, a, b = W.fma_rows_f32((2, 3, 16), seed=4)
    y = REF.stream_ewise("fma", x, a, b, np.float32)
    for i in range(2):
        for r in range(3):
            assert np.array_equal(y[i, r], REF.ewise("fma", [np.full(16, a[i, r]), x[i, r],
                                                             np.full(16, b[i, r])], np.float32))
