"""GPU parity of acp_stream_ewise (the 2..4-stage LDS ring) and of the ring
control itself against the oracle."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import async_copy_pipelining_amd as acp  # noqa: E402
import workloads as W  # noqa: E402
from oracle import reference as REF  # noqa: E402
from oracle import ring as RING  # noqa: E402
from tests.gpu_util import dev, empty_bytes, encode, host, packed_strides, stream, ulp_diff  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", flush=True)


@pytest.mark.parametrize("stages", [1, 2, 3, 4])
def test_ring_trace_matches_oracle_schedule(stages):
    say(f"ring trace stages {stages}")
    for n in range(0, 17):
        # (1,1), (2,1), (2,2), (4,1), (4,4): the compile-time-count ring; the rest the general one
        for loads, stores in ((1, 0), (5, 4), (9, 8), (2, 1), (1, 1), (2, 2), (4, 1), (4, 4)):
            ev = RING.schedule(n, stages, loads, stores)
            out = torch.full((max(1, 3 * n) * 4,), -1, dtype=torch.int32, device="cuda:0")
            acp.acp_debug_ring_trace(n, stages, loads, stores, out, stream())
            got = host(out, np.int32).reshape(-1, 4)[:3 * n]
            want = np.array([[e.kind, e.iteration, e.stage, e.count] for e in ev], dtype=np.int32).reshape(-1, 4)
            assert np.array_equal(got, want), (n, stages, loads, stores)


def _fma_case(shape, stage_box, box, stages, threads, workgroups, seed=4):
    x, a, b = W.fma_rows_f32(shape, seed=seed)
    xd, ad, bd = dev(x), dev(a), dev(b)
    yd = empty_bytes(x.nbytes)
    st = packed_strides(shape)
    xdesc = encode("f32", xd, shape, st, box)
    ydesc = encode("f32", yd, shape, st, box)
    acp.acp_stream_ewise("fma", ydesc, xdesc, ad, bd, stage_box, stages, threads, workgroups, stream())
    return x, a, b, host(yd, np.float32, shape)


@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("workgroups", [0, 8, 5])
def test_c4_small_ragged_fma(stages, workgroups):
    # 37 rows = 9 stages of 4 rows + 1: the last stage is cut; with
    # workgroup tiles of 12 rows two stages of the last tile lie beyond the tensor
    shape, stage_box = (3, 37, 1024), (1, 4, 1024)
    box = (1, 12, 1024) if workgroups == 0 else stage_box
    say(f"C4 small fma {shape} stage {stage_box} box {box} S={stages} wg={workgroups}")
    x, a, b, y = _fma_case(shape, stage_box, box, stages, 256, workgroups)
    ref = REF.stream_ewise("fma", x, a, b, np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("op", ["add", "mul"])
def test_row_add_mul(op):
    shape, stage_box = (2, 9, 512), (1, 2, 512)
    say(f"row {op} {shape} stage {stage_box}")
    x, a, b = W.fma_rows_f32(shape, seed=5)
    xd, ad, bd = dev(x), dev(a), dev(b)
    yd = empty_bytes(x.nbytes)
    st = packed_strides(shape)
    xdesc = encode("f32", xd, shape, st, stage_box)
    ydesc = encode("f32", yd, shape, st, stage_box)
    acp.acp_stream_ewise(op, ydesc, xdesc, ad if op == "mul" else None, bd if op == "add" else None,
                         stage_box, 3, 128, 4, stream())
    ref = REF.stream_ewise(op, x, a, b, np.float32)
    assert np.array_equal(host(yd, np.float32, shape).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("shape,box,stage_box,threads,workgroups,kernel", [
    # a stage spanning two outer indices holds rows 36 (8) apart: the row
    # scalars are staged per row (the scalar-cache path needs consecutive rows)
    ((2, 36, 512), (2, 8, 256), (2, 2, 256), 128, 0, "general stream vec 16 rounds 2 srow 0"),
    ((4, 8, 1024), (2, 4, 1024), (2, 4, 1024), 256, 3, "general stream vec 16 rounds 8 srow 0"),
    # covering the inner row dim whole keeps the stage's rows consecutive
    ((4, 8, 1024), (2, 8, 1024), (2, 8, 1024), 1024, 3, "stream linear grid vec 16 rounds 4 srow 1"),
])
def test_fma_stage_spanning_outer_dims(shape, box, stage_box, threads, workgroups, kernel):
    say(f"fma {shape} box {box} stage {stage_box} threads {threads} wg={workgroups}")
    x, a, b, y = _fma_case(shape, stage_box, box, 3, threads, workgroups, seed=7)
    assert acp.acp_last_kernel().startswith(kernel), acp.acp_last_kernel()
    ref = REF.stream_ewise("fma", x, a, b, np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def test_many_rows_per_stage_and_two_scalar_loads():
    # 48 rows per stage -> two 4-byte row-scalar loads per wave
    shape, stage_box = (2, 100, 64), (1, 48, 64)
    say(f"fma with 48 rows per stage {shape}")
    x, a, b, y = _fma_case(shape, stage_box, stage_box, 3, 256, 0, seed=6)
    ref = REF.stream_ewise("fma", x, a, b, np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


_C4_REF = {}


def _c4_reference(x, a, b):
    """The oracle's streamed fma over the whole [128, 500, 1024] tensor,
    computed once per module (about a second and a half on one core)."""
    if "y" not in _C4_REF:
        _C4_REF["y"] = REF.stream_ewise("fma", x, a, b, np.float32).view(np.uint32)
    return _C4_REF["y"]


@pytest.mark.parametrize("stage_box,stages,threads,workgroups,rounds", [
    ((1, 2, 1024), 4, 256, 256, 2),   # the bench's launch
    ((1, 2, 1024), 3, 256, 256, 2),   # its 3- and 2-stage rings (bench "ring_stages")
    ((1, 2, 1024), 2, 256, 256, 2),
    ((1, 1, 1024), 4, 128, 256, 2),
    ((1, 4, 1024), 4, 256, 512, 4),
    ((1, 4, 1024), 2, 256, 256, 4),
])
def test_c4_full_size_bench_config(stage_box, stages, threads, workgroups, rounds):
    # every element of the full-size streamed fma against the oracle, bit for bit
    shape = (128, 500, 1024)
    say(f"C4 full fma [128,500,1024] stage {stage_box} S={stages} {threads} threads, {workgroups} workgroups")
    x, a, b, y = _fma_case(shape, stage_box, stage_box, stages, threads, workgroups)
    assert acp.acp_last_kernel().startswith(f"stream linear grid vec 16 rounds {rounds} srow 1")
    assert acp.acp_last_kernel().endswith(" xcd-remap")
    assert np.array_equal(y.view(np.uint32), _c4_reference(x, a, b))


@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("rows,workgroups", [(1, 8), (2, 8), (3, 1), (5, 2), (17, 4), (64, 3)])
def test_linear_ring_short_and_long_trip_counts(stages, rows, workgroups):
    # one row per stage on a linear grid: workgroups get 0..22 trips, so the
    # ring runs with no steady state, exactly S-1 trips, and past its warm-up
    shape, stage = (1, rows, 1024), (1, 1, 1024)
    say(f"linear fma {shape} stage {stage} S={stages} workgroups {workgroups}")
    x, a, b, y = _fma_case(shape, stage, stage, stages, 256, workgroups, seed=rows)
    assert acp.acp_last_kernel().startswith("stream linear grid"), acp.acp_last_kernel()
    ref = REF.stream_ewise("fma", x, a, b, np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("k", [2, 3, 5, 9])
def test_general_stream_short_and_long_trip_counts(stages, k):
    # float16 -> float32 sqrt on padded rows with a gap between the outer
    # slices, so the stage grid is not linear and the general kernel runs:
    # each of the two workgroups streams its box's k stages, so the ring runs
    # with no steady state, exactly S-1 trips, and past its warm-up
    shape, pitch, gap = (2, k, 64, 128), 136, 512
    strides = (k * 64 * pitch + gap, 64 * pitch, pitch, 1)
    box, stage = (1, k, 64, 128), (1, 1, 64, 128)
    say(f"general widening stream sqrt {shape} strides {strides} stage {stage} S={stages}")
    rng = np.random.default_rng(20 + k)
    n_store = (shape[0] - 1) * strides[0] + (k - 1) * strides[1] + 63 * pitch + 128
    storage = np.zeros(n_store, np.float16)
    fill = np.lib.stride_tricks.as_strided(storage, shape=shape, strides=tuple(2 * st for st in strides))
    fill[...] = np.abs(rng.standard_normal(shape)).astype(np.float16)
    x = W.strided_view(storage, shape, strides)
    xd = dev(storage)
    n = int(np.prod(shape))
    yd = empty_bytes(n * 4)
    xdesc = encode("f16", xd, shape, strides, box)
    ydesc = encode("f32", yd, shape, packed_strides(shape), box)
    acp.acp_stream_ewise("sqrt", ydesc, xdesc, None, None, stage, stages, 256, 0, stream())
    assert acp.acp_last_kernel().startswith("general stream"), acp.acp_last_kernel()
    y = host(yd, np.float32, shape)
    ref = REF.ewise("sqrt", [np.ascontiguousarray(x)], np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def _exp_table_on_gpu():
    """GPU exp of every float16 in [-4, 4] (34818 values: U(-4, 4) rounded to
    float16 reaches +4.0 as well) through the C5 path."""
    bits = np.concatenate([np.arange(0x0000, 0x4401), np.arange(0x8000, 0xC401)]).astype(np.uint16)
    assert len(bits) == 34818
    rows = -(-len(bits) // 64)
    padded = np.zeros(rows * 64, np.uint16)
    padded[:len(bits)] = bits
    x = padded.view(np.float16).reshape(rows, 64)
    xd = dev(x)
    yd = empty_bytes(x.size * 4)
    xdesc = encode("f16", xd, x.shape, (64, 1), (64, 64), acp.ACP_SWIZZLE_128B)
    ydesc = encode("f32", yd, x.shape, (64, 1), (64, 64))
    acp.acp_stream_ewise("exp", ydesc, xdesc, None, None, (8, 64), 4, 64, 0, stream())
    y = host(yd, np.float32).reshape(-1)[:len(bits)]
    return bits, y


def test_exp_exhaustive_f16_inputs_within_one_ulp():
    say("exp over all 34818 float16 inputs in [-4, 4]")
    bits, y = _exp_table_on_gpu()
    ref = REF.ewise("exp", [bits.view(np.float16)], np.float32)
    d = ulp_diff(y, ref)
    assert d.max() <= 1
    print(f"exp table: {np.count_nonzero(d == 0)} / {len(d)} bit-exact", flush=True)


@pytest.mark.parametrize("mode,threads", [(acp.ACP_SWIZZLE_128B, 256), (acp.ACP_SWIZZLE_64B, 256),
                                          (acp.ACP_SWIZZLE_32B, 256), (acp.ACP_SWIZZLE_32B, 128),
                                          (acp.ACP_SWIZZLE_32B, 512)])
def test_c5_small_rank5_exp(mode, threads):
    # every swizzle mode, at 2, 4 and 1 rounds per wave under the 32-byte one
    shape, pitch = (1, 2, 4, 64, 128), 136
    say(f"C5 small rank-5 exp {shape} pitch {pitch} swizzle {mode} threads {threads}")
    storage, strides = W.padded_uniform_f16(shape, pitch=pitch, seed=5)
    xd = dev(storage)
    n = int(np.prod(shape))
    yd = empty_bytes(n * 4)
    xdesc = encode("f16", xd, shape, strides, (1, 2, 4, 64, 64), mode)
    ydesc = encode("f32", yd, shape, packed_strides(shape), (1, 2, 4, 64, 64))
    acp.acp_stream_ewise("exp", ydesc, xdesc, None, None, (1, 1, 1, 64, 64), 4, threads, 0, stream())
    assert acp.acp_last_kernel().startswith("general stream"), acp.acp_last_kernel()
    y = host(yd, np.float32, shape)
    x = W.strided_view(storage, shape, strides)
    ref = REF.ewise("exp", [x], np.float32)
    assert not np.any(np.isnan(y))
    assert ulp_diff(y.reshape(-1), ref.reshape(-1)).max() <= 1


def test_c5_full_size_matches_exp_table():
    shape, pitch = (4, 8, 64, 128, 256), 264
    say(f"C5 full rank-5 exp {shape} pitch {pitch}, box (1,2,16,64,64), stage (1,1,1,64,64), S=4")
    bits, table = _exp_table_on_gpu()
    lut = torch.zeros(65536, dtype=torch.int32, device="cuda:0")
    lut[torch.from_numpy(bits.astype(np.int64)).cuda()] = torch.from_numpy(table.view(np.int32).copy()).cuda()
    storage, strides = W.padded_uniform_f16(shape, pitch=pitch, seed=5)
    xd = dev(storage)
    n = int(np.prod(shape))
    yd = empty_bytes(n * 4)
    box = (1, 2, 16, 64, 64)
    xdesc = encode("f16", xd, shape, strides, box, acp.ACP_SWIZZLE_128B)
    ydesc = encode("f32", yd, shape, packed_strides(shape), box)
    info = acp.acp_plan_query(xdesc, 256, copy_only=False)
    assert info["rank"] == 5
    acp.acp_stream_ewise("exp", ydesc, xdesc, None, None, (1, 1, 1, 64, 64), 4, 256, 0, stream())
    torch.cuda.synchronize()
    xbits = xd.view(torch.int16).view(-1, pitch)[:, :256].reshape(-1).to(torch.int64) & 0xFFFF
    want = lut[xbits]
    got = yd.view(torch.int32)
    assert torch.equal(got, want)
    assert not torch.isnan(yd.view(torch.float32)).any()


@pytest.mark.parametrize("threads,stage_box,mode", [(256, (1, 2, 64, 128), 3), (256, (1, 1, 64, 128), 3),
                                                    (64, (1, 1, 8, 128), 3), (256, (1, 1, 64, 128), 1),
                                                    (64, (1, 1, 8, 128), 2), (256, (1, 1, 64, 64), 1),
                                                    (512, (1, 1, 64, 128), 1)])
def test_widening_stream_pieces_ragged(threads, stage_box, mode):
    # float16 -> float32 sqrt: 8-byte input pieces, 16-byte stores; 70 rows
    # = 64 + 6 cut the last stage; padded input pitch 136
    shape, pitch = (3, 2, 70, 128), 136
    say(f"widening stream sqrt {shape} stage {stage_box} threads {threads} swizzle mode {mode}")
    storage, strides = W.padded_uniform_f16(shape, pitch=pitch, seed=8)
    storage = np.abs(storage)
    xd = dev(storage)
    n = int(np.prod(shape))
    yd = empty_bytes(n * 4)
    box = (1, 2, 64, 128)
    xdesc = encode("f16", xd, shape, strides, box, mode)
    ydesc = encode("f32", yd, shape, packed_strides(shape), box)
    acp.acp_stream_ewise("sqrt", ydesc, xdesc, None, None, stage_box, 3, threads, 0, stream())
    y = host(yd, np.float32, shape)
    x = W.strided_view(storage, shape, strides)
    ref = REF.ewise("sqrt", [x], np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def _binary_case(op, dt, shape, box, stage_box, stages, threads, workgroups, staging, swizzle=0, seed=41):
    npdt = {"f16": np.float16, "f32": np.float32}[dt]
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(npdt)
    z = rng.standard_normal(shape).astype(npdt)
    xd, zd = dev(x), dev(z)
    yd = empty_bytes(x.nbytes)
    st = packed_strides(shape)
    xdesc = encode(dt, xd, shape, st, box, swizzle)
    zdesc = encode(dt, zd, shape, st, box, swizzle)
    ydesc = encode(dt, yd, shape, st, box)
    acp.acp_stream_binary(op, ydesc, xdesc, zdesc, stage_box, stages, threads, workgroups, staging, stream())
    return x, z, host(yd, npdt, shape)


@pytest.mark.parametrize("staging", ["ring", "set"])
@pytest.mark.parametrize("op,dt,shape,box,stage_box,stages,threads,workgroups,swz", [
    ("add", "f32", (3, 37, 1024), (1, 12, 1024), (1, 4, 1024), 4, 256, 0, 0),   # cut last stage
    ("mul", "f32", (3, 37, 1024), (1, 4, 1024), (1, 4, 1024), 3, 256, 5, 0),    # persistent, uneven
    ("add", "f16", (2, 70, 256), (1, 8, 256), (1, 4, 128), 2, 64, 0, 3),        # swizzled, two loads per trip
    ("mul", "f16", (4, 33, 512), (1, 16, 256), (1, 16, 64), 4, 128, 7, 2),      # 64-byte swizzle, sub-stages
    # full stages on a row-major stage grid: both tensors on the ring run the linear-grid kernel
    ("add", "f32", (3, 36, 1024), (1, 4, 1024), (1, 4, 1024), 3, 256, 5, 0),    # persistent, uneven
    ("mul", "f16", (4, 32, 512), (1, 8, 512), (1, 8, 512), 2, 128, 0, 3),       # swizzled, one tile per workgroup
])
def test_two_tensor_stream_matches_oracle(staging, op, dt, shape, box, stage_box, stages, threads, workgroups, swz):
    say(f"two-tensor stream {op} {dt} {shape} box {box} stage {stage_box} S={stages} wg={workgroups} "
        f"z={staging} swizzle {swz}")
    x, z, y = _binary_case(op, dt, shape, box, stage_box, stages, threads, workgroups, staging, swz)
    kernel = acp.acp_last_kernel()
    linear = box == stage_box and shape[1] % box[1] == 0
    assert kernel.startswith("stream linear grid" if linear and staging == "ring" else "general stream"), kernel
    assert f" variant {1 if staging == 'ring' else 2} " in kernel
    ref = REF.ewise(op, [x, z], y.dtype)
    bits = np.uint16 if dt == "f16" else np.uint32
    assert np.array_equal(y.view(bits), ref.view(bits))


@pytest.mark.parametrize("staging", ["ring", "set"])
def test_two_tensor_stream_full_size(staging):
    shape, stage_box = (128, 500, 1024), (1, 2, 1024)
    say(f"two-tensor stream add {shape} stage {stage_box} S=4, 256 workgroups, z={staging}")
    x, z, y = _binary_case("add", "f32", shape, stage_box, stage_box, 4, 256, 256, staging, seed=42)
    assert acp.acp_last_kernel().startswith("stream linear grid" if staging == "ring" else "general stream")
    ref = REF.ewise("add", [x, z], np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("rows,workgroups", [(1, 8), (3, 1), (5, 2), (17, 4)])
def test_linear_two_tensor_short_and_long_trip_counts(stages, rows, workgroups):
    # x + z with both tensors on the ring (two loads per round) on a linear
    # grid with 0..17 trips per workgroup
    shape, stage = (1, rows, 1024), (1, 1, 1024)
    say(f"linear two-tensor add {shape} stage {stage} S={stages} workgroups {workgroups}")
    x, z, y = _binary_case("add", "f32", shape, stage, stage, stages, 256, workgroups, "ring", seed=80 + rows)
    assert acp.acp_last_kernel().startswith("stream linear grid"), acp.acp_last_kernel()
    assert " variant 1 " in acp.acp_last_kernel()
    ref = REF.ewise("add", [x, z], np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def _reduce_rows_case(dt, shape, box, stage_box, stages, threads, workgroups, ints=False, swz=0, pitch=None, seed=61):
    npdt = {"f16": np.float16, "f32": np.float32}[dt]
    rng = np.random.default_rng(seed)
    if ints:
        x = rng.integers(-50, 51, size=shape).astype(npdt)
    else:
        x = (rng.standard_normal(shape) * 4).astype(npdt)
    st = packed_strides(shape)
    if pitch:                                   # padded rows
        store = np.zeros(shape[:-1] + (pitch,), npdt)
        store[..., :shape[-1]] = x
        xd = dev(store)
        st = packed_strides(shape[:-1] + (pitch,))
    else:
        xd = dev(x)
    rows = int(np.prod(shape[:-1]))
    yd = empty_bytes(rows * 4 + 64)
    xdesc = encode(dt, xd, shape, st, box, swz)
    acp.acp_stream_reduce_rows("add", yd, xdesc, stage_box, stages, threads, workgroups, stream())
    y = host(yd, np.float32)
    assert np.all(y.view(np.uint8)[rows * 4:] == 0xA5)          # nothing written past the rows
    return x, y[:rows].reshape(shape[:-1])


@pytest.mark.parametrize("stages", [2, 3, 4])
@pytest.mark.parametrize("n_stages,workgroups", [(1, 8), (2, 8), (3, 1), (5, 2), (17, 4), (40, 3)])
def test_linear_row_sums_short_and_long_trip_counts(stages, n_stages, workgroups):
    # wave-local row sums on a linear grid with 0..17 trips per workgroup:
    # no steady state, exactly S-1 trips, and past the ring's warm-up
    shape = (1, 4 * n_stages, 1024)
    say(f"linear row sums {shape} stage (1,4,1024) S={stages} workgroups {workgroups}")
    x, y = _reduce_rows_case("f32", shape, (1, 4, 1024), (1, 4, 1024), stages, 256, workgroups, ints=True,
                             seed=70 + n_stages)
    assert acp.acp_last_kernel().startswith("row reduction linear grid"), acp.acp_last_kernel()
    assert np.array_equal(y, REF.reduce_rows(x))


def _assert_within_sum_bound(x, y):
    ref = REF.reduce_rows(x).astype(np.float64)
    bound = REF.recursive_sum_bound(x, x.shape[-1] - 1) + np.spacing(np.abs(ref.astype(np.float32))).astype(np.float64)
    err = np.abs(y.astype(np.float64) - ref)
    assert np.all(err <= bound), float((err - bound).max())


# kernel kinds: the linear-grid kernel (full stages on a row-major stage
# grid, wave-local) and the general kernel, wave-local or through LDS
LIN, LOCAL, LDS = ("row reduction linear grid", "wave-local"), ("general row reduction", "wave-local"), \
    ("general row reduction", "lds partials")


@pytest.mark.parametrize("dt,shape,box,stage_box,stages,threads,workgroups,swz,pitch,kind", [
    # The stage image is issue-major (rows wider than 256 elements load as
    # 256-element segments), so 1 KiB block b of a (1, R, 1024) f32 stage is
    # segment b // R of row b % R and goes to wave b % waves: with R equal
    # to the wave count (or one wave) every row's blocks meet in one wave,
    # which then reduces its rows alone ("wave-local"); otherwise the chunk
    # partials go through LDS behind a workgroup barrier.
    ("f32", (3, 37, 1024), (1, 12, 1024), (1, 4, 1024), 4, 256, 0, 0, None, LOCAL),   # 4 loads per stage, cut stage
    ("f32", (3, 37, 1024), (1, 4, 1024), (1, 4, 1024), 2, 256, 5, 0, None, LOCAL),    # persistent, uneven
    ("f32", (3, 37, 1024), (1, 4, 1024), (1, 2, 1024), 3, 256, 0, 0, None, LDS),      # 2 rows over 4 waves
    ("f16", (2, 70, 256), (1, 8, 256), (1, 8, 256), 3, 64, 5, 3, None, LDS),          # swizzled f16, 8 rows per stage
    ("f32", (5, 64, 64), (1, 16, 64), (1, 16, 64), 4, 64, 0, 0, None, LDS),           # 16 rows per wave block
    ("f32", (4, 33, 96), (1, 8, 96), (1, 8, 96), 3, 192, 0, 0, 104, LDS),             # padded rows, 3 waves
    ("f32", (3, 37, 1024), (1, 4, 1024), (1, 1, 1024), 3, 64, 0, 0, None, LOCAL),     # one wave, 4 stages per tile
    ("f32", (3, 37, 1024), (1, 2, 1024), (1, 2, 1024), 2, 64, 7, 0, None, LOCAL),     # one wave, persistent
    ("f16", (2, 50, 2048), (1, 5, 2048), (1, 1, 2048), 4, 64, 0, 3, None, LOCAL),     # swizzled f16 rows of 4 KiB
    ("f32", (4, 20, 512), (1, 4, 512), (1, 2, 512), 2, 64, 0, 0, None, LOCAL),        # 2 KiB rows, two blocks each
    # full stages on a row-major stage grid: the linear-grid kernel
    ("f32", (3, 36, 1024), (1, 4, 1024), (1, 4, 1024), 2, 256, 5, 0, None, LIN),      # persistent, uneven
    ("f32", (3, 36, 1024), (1, 2, 1024), (1, 2, 1024), 4, 64, 0, 0, None, LIN),       # one wave, 2 rows per stage
    ("f16", (2, 50, 2048), (1, 1, 2048), (1, 1, 2048), 3, 64, 9, 3, None, LIN),       # swizzled f16 rows of 4 KiB
    ("f32", (4, 20, 512), (1, 2, 512), (1, 2, 512), 2, 64, 0, 0, None, LIN),          # 2 KiB rows
    # a 64-byte swizzle splits 2 KiB rows into 64-byte atoms (atom axis
    # outermost), so every 1 KiB block spans both rows of the stage
    ("f32", (4, 20, 512), (1, 2, 512), (1, 2, 512), 2, 64, 0, 2, None, LDS),
    # stage rows 40 apart: the stage grid is not row-major contiguous
    ("f32", (2, 8, 40, 1024), (1, 2, 4, 1024), (1, 2, 4, 1024), 3, 256, 11, 0, None, LOCAL),
])
def test_row_reduction_matches_oracle(dt, shape, box, stage_box, stages, threads, workgroups, swz, pitch, kind):
    say(f"row reduction {dt} {shape} box {box} stage {stage_box} S={stages} wg={workgroups} swz {swz} pitch {pitch}")
    # integer inputs: every partial sum exact, so the result is the exact sum
    x, y = _reduce_rows_case(dt, shape, box, stage_box, stages, threads, workgroups, True, swz, pitch)
    kernel = acp.acp_last_kernel()
    assert kernel.startswith(kind[0]) and kernel.endswith(kind[1]), kernel
    assert np.array_equal(y, REF.reduce_rows(x))
    # real-valued inputs: within the recursive-summation bound of the exact sum
    x, y = _reduce_rows_case(dt, shape, box, stage_box, stages, threads, workgroups, False, swz, pitch, seed=62)
    _assert_within_sum_bound(x, y)


@pytest.mark.parametrize("stage_box,stages,threads,workgroups,kind", [
    ((1, 2, 1024), 4, 256, 256, LDS),
    ((1, 4, 1024), 2, 256, 512, LIN),          # the bench shape
    ((1, 1, 1024), 2, 64, 2048, LIN),
])
def test_row_reduction_full_size(stage_box, stages, threads, workgroups, kind):
    shape = (128, 500, 1024)
    say(f"row reduction f32 {shape} stage {stage_box} S={stages}, {threads} threads, {workgroups} workgroups")
    x, y = _reduce_rows_case("f32", shape, stage_box, stage_box, stages, threads, workgroups, False, seed=63)
    kernel = acp.acp_last_kernel()
    assert kernel.startswith(kind[0]) and kernel.endswith(kind[1]), kernel
    _assert_within_sum_bound(x, y)


def test_repeated_calls_reuse_or_rebuild_their_launch():
    # The library keeps each call's prepared launch, keyed by its arguments:
    # alternating slot counts, thread counts and output buffers (more distinct
    # calls than the per-thread table holds) must each run their own launch.
    shape, stage = (2, 64, 1024), (1, 2, 1024)
    say(f"repeated fma calls {shape} with changing arguments")
    x, a, b = W.fma_rows_f32(shape, seed=21)
    xd, ad, bd = dev(x), dev(a), dev(b)
    st = packed_strides(shape)
    xdesc = encode("f32", xd, shape, st, stage)
    outs = [empty_bytes(x.nbytes) for _ in range(3)]
    ydescs = [encode("f32", o, shape, st, stage) for o in outs]
    ref = REF.stream_ewise("fma", x, a, b, np.float32).view(np.uint32)
    combos = [(s, t, w, k) for s in (2, 3, 4) for t in (128, 256) for w in (4, 8, 16) for k in range(3)]
    for rep in range(2):
        for stages, threads, wgs, k in combos:
            outs[k].fill_(0xA5)
            acp.acp_stream_ewise("fma", ydescs[k], xdesc, ad, bd, stage, stages, threads, wgs, stream())
            kern = acp.acp_last_kernel()
            assert f" grid {wgs} threads {threads} slots {stages} " in kern, kern
            assert np.array_equal(host(outs[k], np.uint32, shape), ref), (rep, stages, threads, wgs, k)


def test_ring_at_the_lds_limit_and_one_row_past_it():
    # four 40 KiB slots take the whole 160 KiB of LDS a workgroup may hold on
    # the MI355X: the ring runs and equals the oracle; 44 KiB slots need
    # 176 KiB and are refused on the host (ACP_ERR_LDS) before any launch.
    # 16 stages over 4 workgroups: 4 trips each, so the ring keeps 4 slots
    shape = (4, 40, 1024)
    say(f"sqrt stream {shape}, stage (1,10,1024) x 4 slots (160 KiB), 640 threads")
    x = np.abs(W.sqrt_tiles_f32(160, seed=71)).reshape(shape)
    xd, yd = dev(x), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    xdesc, ydesc = encode("f32", xd, shape, st, (1, 10, 1024)), encode("f32", yd, shape, st, (1, 10, 1024))
    acp.acp_stream_ewise("sqrt", ydesc, xdesc, None, None, (1, 10, 1024), 4, 640, 4, stream())
    kernel = acp.acp_last_kernel()
    assert " threads 640 slots 4 lds 163840" in kernel, kernel
    want = REF.ewise("sqrt", [x], np.float32).view(np.uint32)
    assert np.array_equal(host(yd, np.float32, shape).view(np.uint32), want)
    shape2 = (4, 44, 1024)
    x2d, y2d = empty_bytes(int(np.prod(shape2)) * 4), empty_bytes(int(np.prod(shape2)) * 4)
    st2 = packed_strides(shape2)
    x2, y2 = encode("f32", x2d, shape2, st2, (1, 11, 1024)), encode("f32", y2d, shape2, st2, (1, 11, 1024))
    with pytest.raises(acp.AcpError) as e:
        acp.acp_stream_ewise("sqrt", y2, x2, None, None, (1, 11, 1024), 4, 704, 4, stream())
    assert e.value.status == acp.ACP_ERR_LDS and "180224" in str(e.value), str(e.value)
