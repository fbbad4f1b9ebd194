"""GPU parity of acp_tile_ewise (operands and output staged in LDS) against
the oracle's elementwise definitions: bit-exact for zero / add / mul / fma /
sqrt, within 1 ulp for exp."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import async_copy_pipelining_amd as acp  # noqa: E402
import workloads as W  # noqa: E402
from oracle import reference as REF  # noqa: E402
from tests.gpu_util import dev, empty_bytes, encode, host, packed_strides, stream, ulp_diff  # noqa: E402

NP = {"f16": np.float16, "f32": np.float32}


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def run_tile_ewise(op, ins, in_dt, out_dt, shape, box, threads, swizzle=0):
    st = packed_strides(shape)
    bufs = [dev(a) for a in ins]
    descs = [encode(in_dt, b, shape, st, box, swizzle) for b in bufs]
    n = int(np.prod(shape))
    yd = empty_bytes(n * np.dtype(NP[out_dt]).itemsize)
    out = encode(out_dt, yd, shape, st, box, swizzle)
    acp.acp_tile_ewise(op, out, descs, threads, stream())
    return host(yd, NP[out_dt], shape)


def test_c2_small_sqrt_bit_exact():
    say("C2 sqrt 96 tiles of 32x32 f32, 256 threads")
    x = W.sqrt_tiles_f32(tiles=96, seed=2)
    y = run_tile_ewise("sqrt", [x], "f32", "f32", x.shape, (1, 32, 32), 256)
    ref = REF.ewise("sqrt", [x], np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def test_c2_full_size_sqrt():
    say("C2 sqrt 65536 tiles of 32x32 f32, 256 threads")
    x = W.sqrt_tiles_f32(tiles=65536, seed=2)
    y = run_tile_ewise("sqrt", [x], "f32", "f32", x.shape, (1, 32, 32), 256)
    assert acp.acp_last_kernel().startswith("tile linear grid vec 16 rounds 4 ")   # 4 tiles per stage
    ref = REF.ewise("sqrt", [x], np.float32)
    d = ulp_diff(y.reshape(-1), ref.reshape(-1))
    assert d.max() <= 1
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))   # correctly rounded in practice


CASES = [
    # op, n_in, in dtype, out dtype, shape, box, threads, swizzle
    ("add", 2, "f32", "f32", (3, 70, 128), (1, 16, 128), 256, 0),
    ("mul", 2, "f32", "f32", (3, 70, 128), (1, 16, 128), 256, 3),
    ("fma", 3, "f32", "f32", (3, 70, 128), (1, 16, 128), 256, 0),
    ("add", 2, "f16", "f16", (2, 50, 256), (1, 8, 256), 128, 3),
    ("mul", 2, "f16", "f16", (2, 50, 256), (1, 8, 256), 128, 0),
    ("fma", 3, "f16", "f16", (2, 50, 256), (1, 8, 256), 128, 0),
    ("zero", 1, "f32", "f32", (3, 70, 128), (1, 16, 128), 256, 0),
    ("sqrt", 1, "f16", "f16", (2, 50, 256), (1, 8, 256), 128, 3),
    ("sqrt", 1, "f16", "f32", (2, 50, 256), (1, 8, 256), 128, 0),
    ("exp", 1, "f32", "f32", (3, 70, 128), (1, 16, 128), 256, 0),
    ("exp", 1, "f16", "f32", (2, 50, 256), (1, 8, 256), 128, 3),
    ("exp", 1, "f32", "f16", (3, 70, 128), (1, 16, 128), 256, 0),
    # eight rounds per thread: three operands consumed in groups of rounds;
    # a widening op past the 8-byte piece consumer's limit
    ("fma", 3, "f32", "f32", (3, 70, 128), (1, 16, 128), 64, 0),
    ("exp", 1, "f16", "f32", (2, 50, 256), (1, 16, 256), 64, 3),
    ("sqrt", 1, "f16", "f32", (2, 50, 256), (1, 8, 256), 64, 3),
    # 32- and 64-byte swizzles
    ("exp", 1, "f16", "f32", (2, 50, 256), (1, 8, 256), 128, 1),
    ("fma", 3, "f32", "f32", (3, 70, 128), (1, 16, 128), 256, 2),
    ("mul", 2, "f16", "f16", (2, 50, 256), (1, 8, 256), 128, 2),
]


@pytest.mark.parametrize("case", CASES, ids=[f"{c[0]}-{c[2]}-{c[3]}-swz{c[7]}" for c in CASES])
def test_tile_ewise_ops(case):
    op, n_in, idt, odt, shape, box, threads, swz = case
    say(f"tile_ewise {op} {idt}->{odt} {shape} box {box} threads {threads} swizzle {swz}")
    rng = np.random.default_rng(21)
    if op == "exp":
        ins = [rng.uniform(-8, 8, shape).astype(NP[idt])]
    elif op == "sqrt":
        ins = [rng.uniform(0, 1e3, shape).astype(NP[idt])]
    else:
        ins = [rng.standard_normal(shape).astype(NP[idt]) for _ in range(n_in)]
    y = run_tile_ewise(op, ins, idt, odt, shape, box, threads, swz)
    ref = REF.ewise(op, ins, NP[odt])
    if op == "exp":
        assert ulp_diff(y.reshape(-1), ref.reshape(-1)).max() <= 1
    else:
        assert np.array_equal(y.view(np.uint32 if odt == "f32" else np.uint16),
                              ref.view(np.uint32 if odt == "f32" else np.uint16))


def test_denormals_survive_fma_and_mul():
    say("denormal results of fma / mul (no flush to zero)")
    shape = (1, 64, 64)
    tiny = np.float32(np.finfo(np.float32).smallest_subnormal)
    a = np.full(shape, 0.5, np.float32)
    b = (np.arange(64 * 64, dtype=np.float32).reshape(shape) % 7 + 1) * tiny * 4
    c = np.zeros(shape, np.float32)
    y = run_tile_ewise("fma", [a, b, c], "f32", "f32", shape, (1, 64, 64), 256)
    assert np.array_equal(y, REF.ewise("fma", [a, b, c], np.float32))
    assert np.count_nonzero(y) == y.size


@pytest.mark.parametrize("op,dt,shape,box,threads", [
    ("fma", "f16", (2500, 16, 64), (1, 16, 64), 64),      # 2500 tiles, uneven over the grid
    ("sqrt", "f32", (12, 1501, 64), (1, 8, 64), 64),      # 188 tiles per batch, the last one 5 rows
    ("sqrt", "f32", (31, 333, 500), (1, 16, 16), 64),     # 64-byte rows: two tiles per ring trip
    ("exp", "f16", (20, 333, 1000), (1, 32, 16), 64),     # widening (f16 -> f32), two tiles per trip
])
def test_persistent_grid_ragged_tile_ewise(op, dt, shape, box, threads):
    say(f"persistent tile_ewise {op} {dt} {shape} box {box} threads {threads}")
    if op == "fma":
        ins = [W.normal_f16(shape, seed=s) for s in (21, 22, 23)]
    elif op == "exp":
        ins = [W.normal_f16(shape, seed=25)]
    else:
        ins = [np.abs(W.fma_rows_f32(shape, seed=24)[0])]
    odt = "f32" if op == "exp" else dt
    y = run_tile_ewise(op, ins, dt, odt, shape, box, threads)
    ref = REF.ewise(op, ins, NP[odt])
    if op == "exp":
        assert ulp_diff(y.reshape(-1), ref.reshape(-1)).max() <= 1
    else:
        assert np.array_equal(y.view(np.uint16 if dt == "f16" else np.uint32),
                              ref.view(np.uint16 if dt == "f16" else np.uint32))


@pytest.mark.parametrize("op,shape,box,threads", [
    ("sqrt", (600, 32, 32), (1, 32, 32), 256),            # persistent grid, four tiles per trip
    ("fma", (3, 70, 128), (1, 16, 128), 256),             # one workgroup per tile, ragged last tile
])
def test_tile_ewise_in_place(op, shape, box, threads):
    """The output may be an operand element for element: every element is
    staged before the same lane stores its result, and no other trip
    touches it."""
    say(f"in-place tile_ewise {op} {shape} box {box} threads {threads}")
    rng = np.random.default_rng(26)
    if op == "sqrt":
        ins = [rng.uniform(0, 1e3, shape).astype(np.float32)]
    else:
        ins = [rng.standard_normal(shape).astype(np.float32) for _ in range(3)]
    st = packed_strides(shape)
    bufs = [dev(a) for a in ins]
    descs = [encode("f32", b, shape, st, box) for b in bufs]
    acp.acp_tile_ewise(op, descs[0], descs, threads, stream())
    y = host(bufs[0], np.float32, shape)
    assert np.array_equal(y.view(np.uint32), REF.ewise(op, ins, np.float32).view(np.uint32))


@pytest.mark.parametrize("op,n_in,idt,odt,shape,box,threads,swz,rounds", [
    ("fma", 3, "f32", "f32", (4, 64, 128), (1, 16, 128), 256, 0, 2),      # one workgroup per tile
    ("exp", 1, "f16", "f32", (2, 64, 256), (1, 8, 256), 128, 3, 2),       # widening, swizzled
    ("sqrt", 1, "f32", "f16", (4, 64, 128), (1, 16, 128), 256, 0, 2),     # narrowing
    ("add", 2, "f16", "f16", (8, 32, 64), (1, 32, 64), 64, 2, 4),         # 64-byte swizzle
    ("mul", 2, "f32", "f32", (2048, 32, 32), (1, 32, 32), 256, 0, 2),     # persistent, 2 tiles per stage
    ("exp", 1, "f16", "f32", (1024, 32, 64), (1, 32, 64), 256, 3, 4),     # persistent, 4 tiles per stage
    ("sqrt", 1, "f32", "f32", (1026, 32, 32), (1, 32, 32), 256, 0, 2),    # 1026 tiles: 2 per stage
    ("sqrt", 1, "f16", "f16", (32, 65536), (32, 64), 256, 1, 4),          # tiles 128 B apart in memory
])
def test_tile_ewise_on_a_linear_tile_grid(op, n_in, idt, odt, shape, box, threads, swz, rounds):
    """Full tiles on a row-major tile grid run the linear kernel: the tiles
    of a ring trip form one stage, the output goes through the LDS image."""
    say(f"linear-grid tile_ewise {op} {idt}->{odt} {shape} box {box} threads {threads} swizzle {swz}")
    rng = np.random.default_rng(27)
    if op == "exp":
        ins = [rng.uniform(-8, 8, shape).astype(NP[idt])]
    elif op == "sqrt":
        ins = [rng.uniform(0, 1e3, shape).astype(NP[idt])]
    else:
        ins = [rng.standard_normal(shape).astype(NP[idt]) for _ in range(n_in)]
    y = run_tile_ewise(op, ins, idt, odt, shape, box, threads, swz)
    kernel = acp.acp_last_kernel()
    assert kernel.startswith(f"tile linear grid vec 16 rounds {rounds} "), kernel
    ref = REF.ewise(op, ins, NP[odt])
    if op == "exp":
        assert ulp_diff(y.reshape(-1), ref.reshape(-1)).max() <= 1
    else:
        bits = np.uint32 if odt == "f32" else np.uint16
        assert np.array_equal(y.view(bits), ref.view(bits))


@pytest.mark.parametrize("tiles", [516, 1028, 2052, 5124])
def test_linear_tile_sqrt_short_and_long_trip_counts(tiles):
    # a persistent linear tile grid (4 tiles per stage, one workgroup per CU)
    # with 0..6 trips per workgroup
    x = W.sqrt_tiles_f32(tiles=tiles, seed=tiles)
    shape, box = x.shape, (1, 32, 32)
    say(f"linear tile sqrt {shape}")
    xd = dev(x)
    yd = empty_bytes(x.nbytes)
    st = packed_strides(shape)
    acp.acp_tile_ewise("sqrt", encode("f32", yd, shape, st, box), [encode("f32", xd, shape, st, box)], 256, stream())
    assert acp.acp_last_kernel().startswith("tile linear grid"), acp.acp_last_kernel()
    y = host(yd, np.float32, shape)
    ref = REF.ewise("sqrt", [x], np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))
