"""GPU parity of acp_tile_copy and the direct-to-LDS image against the oracle.

Copy must be bit-identical to its input (the plain definition); the raw LDS
bytes of a staged tile must equal the oracle's swizzled, zero-filled image.
"""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import async_copy_pipelining_amd as acp  # noqa: E402
import workloads as W  # noqa: E402
from oracle import plan as P  # noqa: E402
from oracle import reference as REF  # noqa: E402
from oracle import tiles as T  # noqa: E402
from tests.gpu_util import dev, empty_bytes, encode, host, packed_strides, stream  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _lds_image(desc, tile, threads, nbytes):
    out = empty_bytes(nbytes, 0x5A)
    acp.acp_debug_lds_image(desc, tile, threads, out, stream())
    return host(out, np.uint8)[:nbytes].tobytes()


def test_c1_swizzled_copy_is_bit_identical_and_image_matches():
    say("C1 8x256 f16 swizzled copy, 64 threads")
    x = W.tile_bits_f16((8, 256), seed=1)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    src = encode("f16", xd, (8, 256), (256, 1), (8, 256), acp.ACP_SWIZZLE_128B)
    dst = encode("f16", yd, (8, 256), (256, 1), (8, 256), acp.ACP_SWIZZLE_128B)
    info = acp.acp_plan_query(src, 64)
    assert (info["rank"], info["vec"], info["outer"]) == (3, 8, 4)
    acp.acp_tile_copy(src, dst, 64, stream())
    assert acp.acp_last_kernel().startswith("copy linear grid vec 16 rounds 4 "), acp.acp_last_kernel()
    assert np.array_equal(host(yd, np.uint16), x.view(np.uint16).reshape(-1))
    p = P.plan("f16", (8, 256), (256, 1), (8, 256), P.SWIZZLE_128B, threads=64)
    assert _lds_image(src, 0, 64, 4096) == T.lds_image(x.reshape(-1), p, 0)


@pytest.mark.parametrize("dt,shape,box,swz,threads,kind", [
    ("f32", (300, 32, 32), (1, 32, 32), 0, 256, "copy linear grid vec 16 rounds 1 "),      # persistent, 300 tiles
    ("f32", (513, 32, 32), (1, 32, 32), 0, 128, "copy linear grid vec 16 rounds 2 "),      # persistent, ragged
    ("f16", (7, 8, 256), (1, 8, 256), 3, 64, "copy linear grid vec 16 rounds 4 "),        # one workgroup per tile
    ("f16", (3, 16, 256), (1, 16, 256), 3, 128, "copy linear grid vec 16 rounds 4 "),     # two atoms per row
    ("f32", (2, 64, 32), (1, 64, 32), 1, 64, "copy linear grid vec 16 rounds 8 "),        # 32-byte swizzle
    ("f16", (3, 300, 96), (1, 128, 32), 0, 128, "general copy"),                          # ragged: general kernel
    ("f16", (38400, 64), (128, 32), 0, 128, "copy linear grid vec 16 rounds 8 "),         # paired tiles: whole rows
])
def test_linear_grid_tile_copies(dt, shape, box, swz, threads, kind):
    # tile copies whose tiles form a contiguous row-major grid run on the
    # linear kernel: bit-identical, one workgroup per tile or persistent
    say(f"linear-grid copy {dt} {shape} box {box} swizzle {swz} threads {threads}")
    npdt = {"f16": np.uint16, "f32": np.uint32}[dt]
    rng = np.random.default_rng(37)
    x = rng.integers(0, 2 ** (8 * np.dtype(npdt).itemsize), size=shape, dtype=np.uint64).astype(npdt)
    xd, yd = dev(x), empty_bytes(x.nbytes + 64, 0x5A)
    st = packed_strides(shape)
    src = encode(dt, xd, shape, st, box, swz)
    dst = encode(dt, yd, shape, st, box, swz)
    acp.acp_tile_copy(src, dst, threads, stream())
    kernel = acp.acp_last_kernel()
    assert kernel.startswith(kind), kernel
    # persistent grids of contiguous tiles keep the XCD remap; one workgroup
    # per tile (grid below 16 or not a multiple of 8) has none
    assert kernel.endswith(" xcd-remap") == (" grid 256 " in kernel), kernel
    y = host(yd, np.uint8)
    assert np.array_equal(y[:x.nbytes].view(npdt).reshape(shape), x)
    assert np.all(y[x.nbytes:] == 0x5A)


@pytest.mark.parametrize("threads", [64, 128, 256])
def test_ragged_copy_small_and_partial_tile_image(threads):
    shape, box = (3, 300, 96), (1, 128, 32)   # rows 300 = 2 * 128 + 44, several tiles
    say(f"ragged copy {shape} box {box} threads {threads}")
    x = W.normal_f16(shape, seed=3)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    src = encode("f16", xd, shape, st, box)
    dst = encode("f16", yd, shape, st, box)
    acp.acp_tile_copy(src, dst, threads, stream())
    assert np.array_equal(host(yd, np.uint16, shape), x.view(np.uint16))
    p = P.plan("f16", shape, st, box, threads=threads)
    grid = P.tile_grid(shape, box)
    for tc in [(0, 0, 0), (1, 2, 1), (2, 2, 2)]:              # full, partial rows, partial rows
        t = int(np.ravel_multi_index(tc, grid))
        assert _lds_image(src, t, threads, p.tile_bytes) == T.lds_image(x.reshape(-1), p, t)


def test_c3_full_size_copy():
    shape, box = (128, 500, 1024), (1, 128, 32)
    say(f"C3 full copy {shape} box {box} 128 threads")
    x = W.normal_f16(shape, seed=3)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    src = encode("f16", xd, shape, st, box)
    dst = encode("f16", yd, shape, st, box)
    info = acp.acp_plan_query(src, 128)
    assert (info["vec"], info["vec_bytes"], info["outer"]) == (8, 16, 4)
    assert info["n_tiles"] == 128 * 4 * 32
    acp.acp_tile_copy(src, dst, 128, stream())
    torch.cuda.synchronize()
    assert torch.equal(xd, yd)
    # pairs of tiles per trip (128-byte rows, 8 rounds), whole lines: blocked
    # runs of consecutive pairs per workgroup, no XCD remap
    kernel = acp.acp_last_kernel()
    assert kernel.startswith("general copy vec 16 rounds 8 ") and kernel.endswith(" blocked-walk"), kernel


@pytest.mark.parametrize("mode", [1, 2, 3])
def test_swizzled_multi_atom_tiles_and_strided_output(mode):
    shape, box = (5, 40, 512), (1, 16, 256)     # swizzle splits 512-byte rows into atoms; rows ragged
    say(f"swizzle mode {mode} copy {shape} box {box} into a padded output")
    x = W.normal_f16(shape, seed=7)
    xd = dev(x)
    opitch = 520
    ost = (40 * opitch, opitch, 1)
    yd = empty_bytes(5 * 40 * opitch * 2, 0x00)
    src = encode("f16", xd, shape, packed_strides(shape), box, mode)
    dst = encode("f16", yd, shape, ost, box)
    acp.acp_tile_copy(src, dst, 256, stream())
    y = host(yd, np.uint16).reshape(5, 40, opitch)
    assert np.array_equal(y[:, :, :512], x.view(np.uint16))
    assert not np.any(y[:, :, 512:])                        # the pitch padding was never written
    p = P.plan("f16", shape, packed_strides(shape), box, mode, threads=256)
    t = int(np.ravel_multi_index((4, 2, 1), P.tile_grid(shape, box)))
    assert _lds_image(src, t, 256, p.tile_bytes) == T.lds_image(x.reshape(-1), p, t)


@pytest.mark.parametrize("mode,dt,shape,box,threads", [
    (1, "f16", (8, 256), (8, 256), 64),      # 32-byte atoms, 16 of them
    (2, "f16", (8, 256), (8, 256), 64),      # 64-byte atoms
    (1, "f32", (24, 40), (8, 8), 64),        # inner box of one 32-byte atom, no split
    (2, "u8", (16, 192), (16, 64), 64),      # a 64-byte u8 row
])
def test_narrow_swizzle_images_and_copies(mode, dt, shape, box, threads):
    say(f"swizzle mode {mode} {dt} {shape} box {box} threads {threads}")
    rng = np.random.default_rng(12)
    es = P.ESIZE[dt]
    x = rng.integers(0, 256, size=int(np.prod(shape)) * es, dtype=np.uint8)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    src = encode(dt, xd, shape, st, box, mode)
    dst = encode(dt, yd, shape, st, box, mode)
    acp.acp_tile_copy(src, dst, threads, stream())
    assert np.array_equal(host(yd, np.uint8), x)
    p = P.plan(dt, shape, st, box, mode, threads=threads)
    elems = x.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[es])
    for t in range(min(3, int(np.prod(P.tile_grid(shape, box))))):
        assert _lds_image(src, t, threads, p.tile_bytes) == T.lds_image(elems, p, t)


@pytest.mark.parametrize("mode,dt,shape,box,threads", [
    (3, "f16", (16, 96), (16, 96), 64),      # 192-byte rows: shrunk into two 96-byte loads
    (3, "f16", (20, 200), (8, 128), 128),    # 256-byte box over 400-byte rows: two 128-byte loads
    (1, "f16", (16, 24), (16, 24), 64),      # 48-byte rows under the 32-byte mode: three 16-byte loads
    (2, "f32", (32, 36), (16, 36), 192),     # 144-byte rows under the 64-byte mode: three 48-byte loads
    (3, "f16", (8, 4, 12), (8, 4, 12), 64),  # 24-byte rows: four merge into 96 bytes of whole chunks
])
def test_swizzle_shrunk_inner_box(mode, dt, shape, box, threads):
    # "copy_async -> tma", "Algorithm" step 2: an innermost box that does not
    # fit the swizzle atom is shrunk (cut into loads that do) instead of
    # declined; rows narrower than 16 bytes merge up to whole chunks
    say(f"swizzle mode {mode} shrink {dt} {shape} box {box} threads {threads}")
    rng = np.random.default_rng(13)
    es = P.ESIZE[dt]
    x = rng.integers(0, 256, size=int(np.prod(shape)) * es, dtype=np.uint8)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    src = encode(dt, xd, shape, st, box, mode)
    dst = encode(dt, yd, shape, st, box, mode)
    p = P.plan(dt, shape, st, box, mode, threads=threads)
    info = acp.acp_plan_query(src, threads)
    assert (info["issues"], info["vec_bytes"], info["outer"]) == (p.issues, p.vec_bytes, p.outer)
    acp.acp_tile_copy(src, dst, threads, stream())
    assert np.array_equal(host(yd, np.uint8), x)
    elems = x.view({1: np.uint8, 2: np.uint16, 4: np.uint32}[es])
    n = int(np.prod(P.tile_grid(shape, box)))
    for t in sorted({0, n // 2, n - 1}):
        assert _lds_image(src, t, threads, p.tile_bytes) == T.lds_image(elems, p, t)


@pytest.mark.parametrize("shape,box,threads", [
    ((40, 130, 96), (1, 64, 32), 128),       # three tiles per row: the second pair holds one tile
    ((6, 300, 1000), (1, 128, 32), 128),     # 1000 = 31 * 32 + 8: the last tile of a row is cut
    ((8, 64, 256), (1, 16, 16), 64),         # 32-byte rows: four tiles per trip
    ((19, 300, 320), (1, 128, 32), 128),     # 285 pairs over 256 workgroups: runs of two, the last one short
])
def test_paired_tiles_per_trip(shape, box, threads):
    # a persistent copy of tiles narrower than a cache line stages
    # neighbouring tiles side by side in one trip; the output is the input,
    # and the padding of a strided destination is never written
    say(f"paired-tile copy {shape} box {box} threads {threads}")
    x = W.normal_f16(shape, seed=9)
    xd = dev(x)
    pitch = shape[-1] + 24
    ost = (shape[1] * pitch, pitch, 1)
    yd = empty_bytes(shape[0] * shape[1] * pitch * 2, 0x00)
    src = encode("f16", xd, shape, packed_strides(shape), box)
    dst = encode("f16", yd, shape, ost, box)
    acp.acp_tile_copy(src, dst, threads, stream())
    kernel = acp.acp_last_kernel()
    if shape == (19, 300, 320):
        assert kernel.endswith(" blocked-walk"), kernel
    y = host(yd, np.uint16).reshape(shape[0], shape[1], pitch)
    assert np.array_equal(y[:, :, :shape[-1]], x.view(np.uint16))
    assert not np.any(y[:, :, shape[-1]:])


@pytest.mark.parametrize("misalign", [4, 8])
def test_four_byte_path_when_only_4_or_8_aligned(misalign):
    shape, box = (64, 256), (64, 32)
    say(f"4-byte direct-to-LDS path, base misaligned by {misalign}")
    x = W.normal_f16(shape, seed=8)
    xd = empty_bytes(x.nbytes + 64)
    xd[misalign:misalign + x.nbytes] = dev(x)
    yd = empty_bytes(x.nbytes + 64)
    st = packed_strides(shape)
    src = encode("f16", xd, shape, st, box, offset_bytes=misalign)
    dst = encode("f16", yd, shape, st, box, offset_bytes=misalign)
    info = acp.acp_plan_query(src, 128)
    assert info["vec_bytes"] == 4
    acp.acp_tile_copy(src, dst, 128, stream())
    y = host(yd, np.uint8)
    assert np.array_equal(y[misalign:misalign + x.nbytes].view(np.uint16), x.view(np.uint16).reshape(-1))
    assert np.all(y[:misalign] == 0xA5) and np.all(y[misalign + x.nbytes:] == 0xA5)


@pytest.mark.parametrize("dt,np_dt", [("u8", np.uint8), ("u64", np.uint64), ("u32", np.uint32)])
def test_other_element_types(dt, np_dt):
    shape, box = (7, 33, 128), (2, 8, 128)
    say(f"copy {dt} {shape} box {box}")
    rng = np.random.default_rng(9)
    x = rng.integers(0, 255, size=int(np.prod(shape)) * np.dtype(np_dt).itemsize, dtype=np.uint8)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    src = encode(dt, xd, shape, st, box)
    dst = encode(dt, yd, shape, st, box)
    acp.acp_tile_copy(src, dst, 256, stream())
    assert np.array_equal(host(yd, np.uint8), x)


def test_box_larger_than_tensor_and_empty_tensor():
    say("box larger than the tensor; empty tensor")
    x = W.normal_f16((3, 40), seed=10)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    src = encode("f16", xd, (3, 40), (40, 1), (8, 64))
    dst = encode("f16", yd, (3, 40), (40, 1), (8, 64))
    acp.acp_tile_copy(src, dst, 64, stream())
    assert np.array_equal(host(yd, np.uint16, (3, 40)), x.view(np.uint16))
    p = P.plan("f16", (3, 40), (40, 1), (8, 64), threads=64)
    assert _lds_image(src, 0, 64, p.tile_bytes) == T.lds_image(x.reshape(-1), p, 0)
    e = encode("f16", xd, (0, 40), (40, 1), (8, 64))
    f = encode("f16", yd, (0, 40), (40, 1), (8, 64))
    acp.acp_tile_copy(e, f, 64, stream())                     # no tiles: returns without a launch
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape,box,threads", [
    ((3001, 16, 64), (1, 16, 64), 128),        # 3001 whole tiles: more than one per workgroup, uneven
    ((7, 1333, 256), (1, 4, 256), 64),         # 334 tiles per batch, the last one a single row
    ((4100, 2, 512), (1, 2, 512), 64),         # swizzled copy below
    ((41, 333, 1000), (1, 32, 16), 64),        # 32-byte rows: two tiles per ring trip; 28 413 tiles (odd),
                                               # cut rows (333) and a cut last column tile (1000 = 62 * 16 + 8)
])
def test_persistent_grid_ragged_tile_counts(shape, box, threads):
    swz = acp.ACP_SWIZZLE_128B if shape[0] == 4100 else acp.ACP_SWIZZLE_NONE
    say(f"persistent copy {shape} box {box} threads {threads} swizzle {swz}")
    x = W.normal_f16(shape, seed=11)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    src = encode("f16", xd, shape, st, box, swz)
    dst = encode("f16", yd, shape, st, box, swz)
    info = acp.acp_plan_query(src, threads)
    assert info["n_tiles"] > 2048       # beyond one tile per workgroup of the persistent grid
    assert info["vec_bytes"] == 16
    acp.acp_tile_copy(src, dst, threads, stream())
    torch.cuda.synchronize()
    assert torch.equal(xd, yd)


@pytest.mark.parametrize("nbytes,workgroups", [(16, 0), (16384 * 3 + 48, 2), (5_000_000 - 16 * 7, 0)])
def test_reference_stream_copy_is_bit_identical(nbytes, workgroups):
    say(f"reference stream copy of {nbytes} bytes, workgroups {workgroups}")
    rng = np.random.default_rng(31)
    x = rng.integers(0, 256, nbytes + 64, dtype=np.uint8)
    xd = dev(x)
    yd = empty_bytes(nbytes + 64, 0x5A)
    acp.acp_debug_stream_copy(yd, xd, nbytes, workgroups, stream())
    y = host(yd, np.uint8)
    assert np.array_equal(y[:nbytes], x[:nbytes])
    assert np.all(y[nbytes:] == 0x5A)      # nothing written past the end


COPY_SHAPES = [(64, 16), (128, 8), (256, 2), (256, 4), (256, 8), (512, 2), (512, 4), (512, 8), (1024, 2),
               (1024, 4)]


def test_reference_copy_shapes_are_bit_identical():
    # every built shape and cache-policy pair of the copy sweep moves exactly
    # the requested bytes: a short last block, grids below and above the
    # block count
    nbytes = (1 << 20) + 16 * 37
    say(f"reference copy shapes over {nbytes} bytes")
    rng = np.random.default_rng(32)
    x = rng.integers(0, 256, nbytes + 64, dtype=np.uint8)
    xd = dev(x)
    for threads, unroll in COPY_SHAPES:
        for lnt, snt in ((1, 1), (1, 0), (0, 1), (0, 0)):
            for wgs in (0, 3, 4096):
                yd = empty_bytes(nbytes + 64, 0x5A)
                acp.acp_debug_stream_copy_shape(yd, xd, nbytes, wgs, threads, unroll, lnt, snt, stream())
                y = host(yd, np.uint8)
                assert np.array_equal(y[:nbytes], x[:nbytes]), (threads, unroll, lnt, snt, wgs)
                assert np.all(y[nbytes:] == 0x5A), (threads, unroll, lnt, snt, wgs)


def test_reference_copy_shape_rejects_unbuilt_shapes():
    xd, yd = empty_bytes(4096, 1), empty_bytes(4096, 2)
    with pytest.raises(acp.AcpError) as e:
        acp.acp_debug_stream_copy_shape(yd, xd, 4096, 0, 256, 3, 1, 1, stream())
    assert e.value.status == acp.ACP_ERR_UNSUPPORTED
    with pytest.raises(acp.AcpError) as e:
        acp.acp_debug_stream_copy_shape(yd, xd, 4096, 0, 256, 4, 2, 1, stream())
    assert e.value.status == acp.ACP_ERR_INVALID
    assert np.all(host(yd, np.uint8) == 2)


@pytest.mark.parametrize("shape,pitch,box,tpt,threads,wgs", [
    ((3, 300, 320), 336, (1, 128, 32), 2, 128, 0),     # ragged rows; five whole pairs per tile row
    ((2, 130, 352), 352, (1, 128, 32), 2, 128, 7),     # eleven tiles: the last pair is one tile wide
    ((5, 130, 352), 352, (1, 128, 32), 2, 128, 9),     # 60 pairs in runs of 7 over 9 workgroups, the last short
    ((2, 77, 96), 104, (1, 64, 32), 1, 128, 5),         # one tile per group, 64-byte rows
    ((1, 40, 512), 512, (1, 16, 64), 4, 256, 0),        # four tiles per group, 512-byte rows
])
def test_reference_tiled_copy_walk(shape, pitch, box, tpt, threads, wgs):
    # the same-walk copy reference moves every element of a strided f16
    # source into a packed output (row padding never read) and writes
    # nothing past it
    say(f"reference tiled copy {shape} pitch {pitch} box {box} x{tpt}, {threads} threads, wgs {wgs}")
    rng = np.random.default_rng(36)
    storage = rng.integers(0, 2**16, size=(shape[0], shape[1], pitch), dtype=np.uint64).astype(np.uint16)
    xd = dev(storage)
    n = int(np.prod(shape))
    yd = empty_bytes(n * 2 + 64, 0x5A)
    acp.acp_debug_copy_tiles(yd, xd, 2, shape, (shape[1] * pitch, pitch, 1), box, tpt, threads, wgs, stream())
    y = host(yd, np.uint8)
    assert np.array_equal(y[:n * 2].view(np.uint16).reshape(shape), storage[:, :, :shape[2]])
    assert np.all(y[n * 2:] == 0x5A)


def _reduce_case(dt, src_shape, dst_shape, box, threads, values, swz=0, seed=51):
    npdt = {"u32": np.uint32, "f32": np.float32, "f16": np.float16}[dt]
    rng = np.random.default_rng(seed)
    if values == "wide":
        src = rng.integers(0, 2**32, size=src_shape, dtype=np.uint64).astype(np.uint32)
        dst = rng.integers(0, 2**32, size=dst_shape, dtype=np.uint64).astype(np.uint32)
    elif values == "normal":
        src = rng.standard_normal(src_shape).astype(npdt)
        dst = rng.standard_normal(dst_shape).astype(npdt)
    else:                                   # small integers: every partial sum exact
        src = rng.integers(-values, values + 1, size=src_shape).astype(npdt)
        dst = rng.integers(-values, values + 1, size=dst_shape).astype(npdt)
    sd, dd = dev(src), dev(dst)
    sdesc = encode(dt, sd, src_shape, packed_strides(src_shape), box, swz)
    ddesc = encode(dt, dd, dst_shape, packed_strides(dst_shape), box)
    acp.acp_tile_reduce("add", ddesc, sdesc, threads, stream())
    kernel = acp.acp_last_kernel()
    if src_shape == dst_shape and dt != "u32":                                   # ring path, no atomics
        assert kernel.startswith(("general stream", "stream linear grid")) and " variant 1 " in kernel
    elif src_shape != dst_shape:
        assert kernel.startswith("general reduce-add"), kernel
    got = host(dd, npdt, dst_shape)
    want = REF.tile_reduce_add(dst, src)
    bits = {np.uint32: np.uint32, np.float32: np.uint32, np.float16: np.uint16}[npdt]
    return got.view(bits), want.view(bits)


@pytest.mark.parametrize("dt,src_shape,dst_shape,box,threads,values,swz", [
    ("u32", (6, 40, 256), (1, 40, 256), (1, 8, 256), 128, "wide", 0),        # wraps modulo 2**32; cut rows
    ("f32", (3, 37, 128), (3, 37, 128), (1, 8, 128), 64, "normal", 0),       # one contribution: IEEE add (ring path)
    ("f16", (700, 8, 64), (700, 8, 64), (1, 8, 64), 64, "normal", 2),        # one contribution, persistent, swizzled
    ("u32", (3, 37, 128), (3, 37, 128), (1, 8, 128), 64, "wide", 0),         # one contribution, integer: atomics
    ("f32", (16, 33, 64), (1, 33, 64), (1, 8, 64), 64, 100, 3),              # 16 contributions, swizzled staging
    ("f16", (8, 20, 128), (1, 20, 128), (1, 4, 128), 64, 8, 0),              # packed f16 pairs
    ("f32", (600, 16, 64), (1, 16, 64), (1, 16, 64), 64, 4, 0),              # 600 tiles into one: persistent grid
    ("u32", (4, 5, 16, 64), (1, 1, 16, 64), (1, 1, 16, 64), 64, "wide", 0),  # two reduced dims
    ("u32", (3, 7, 40, 64), (3, 1, 40, 64), (1, 1, 8, 64), 64, "wide", 0),   # a middle dim reduced
    ("f32", (2, 2048, 8, 64), (1, 2048, 8, 64), (1, 1, 8, 64), 64, 1000, 0), # more destination tiles than workgroups
    ("f16", (5, 3, 24, 128), (1, 3, 24, 128), (1, 1, 8, 128), 64, 8, 3),     # f16 sums in binary32 registers
])
def test_store_with_reduce_add(dt, src_shape, dst_shape, box, threads, values, swz):
    say(f"reduce-add {dt} {src_shape} -> {dst_shape} box {box} threads {threads} swizzle {swz}")
    got, want = _reduce_case(dt, src_shape, dst_shape, box, threads, values, swz)
    assert np.array_equal(got, want)


def test_reference_read_and_fill_streams():
    # the one-direction measurement references: the read stream's per-
    # workgroup XORs fold to the XOR of every 16-byte word of the source;
    # the fill writes its pattern over exactly the requested bytes
    n = (9 << 20) + 4096 + 48                     # a short last block; 577 blocks of 16 KiB
    say(f"reference read / fill streams over {n} bytes")
    rng = np.random.default_rng(31)
    x = rng.integers(0, 2**32, size=n // 4, dtype=np.uint64).astype(np.uint32)
    xd = dev(x)
    for wgs in (0, 7, 300, 512):                  # 512: two per CU, as the bench's read reference
        sums = empty_bytes(16 * 512, 0x00)
        acp.acp_debug_stream_read(xd, n, sums, wgs, stream())
        g = wgs or 256
        g = min(g, (n + 16383) // 16384)
        got = np.bitwise_xor.reduce(host(sums, np.uint32).reshape(-1, 4)[:g], axis=0)
        want = np.bitwise_xor.reduce(x.reshape(-1, 4), axis=0)
        assert np.array_equal(got, want), wgs
    yd = empty_bytes(n + 64, 0x11)
    acp.acp_debug_stream_fill(yd, n, 0xDEADBEEF, 5, stream())
    y = host(yd, np.uint8)
    assert np.all(y[:n].view(np.uint32) == 0xDEADBEEF) and np.all(y[n:] == 0x11)


def test_reference_widening_stream():
    # the widening reference converts float16 to float32 exactly and writes
    # nothing past the output
    n = (1 << 20) + 8 * 37                   # a short last block
    say(f"reference widening stream over {n} elements")
    x = W.normal_f16((n,), seed=33)
    xd = dev(x)
    yd = empty_bytes(n * 4 + 64, 0x11)
    acp.acp_debug_stream_widen(yd, xd, n, 0, stream())
    y = host(yd, np.uint8)
    assert np.array_equal(y[:n * 4].view(np.float32), x.astype(np.float32))
    assert np.all(y[n * 4:] == 0x11)


@pytest.mark.parametrize("shape,box,stage", [
    ((2, 4, 16, 128, 256), (1, 2, 16, 64, 64), (1, 1, 1, 64, 64)),   # the rank-5 exp walk, reduced
    ((1, 2, 3, 40, 96), (1, 1, 3, 20, 48), (1, 1, 1, 10, 48)),       # 12 pieces per row, 120 per stage
])
def test_reference_widening_tile_walk(shape, box, stage):
    # the same-walk widening reference converts every element exactly into a
    # packed float32 output (row pitch 264 on the input: padding never read)
    say(f"reference tiled widening {shape} box {box} stage {stage}")
    storage, strides = W.padded_uniform_f16(shape, pitch=shape[-1] + 8, seed=34)
    n = int(np.prod(shape))
    xd, yd = dev(storage), empty_bytes(n * 4 + 64, 0x11)
    acp.acp_debug_widen_tiles(yd, xd, shape, strides, box, stage, stream())
    y = host(yd, np.uint8)
    want = W.strided_view(storage, shape, strides).astype(np.float32)
    assert np.array_equal(y[:n * 4].view(np.float32).reshape(shape), want)
    assert np.all(y[n * 4:] == 0x11)
