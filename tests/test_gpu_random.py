"""Seeded random configurations of every pipelined entry point against the
oracle: ranks 2-4, ragged extents (cut last tiles and stages), padded rows,
every swizzle mode, 64-256 threads, 1-4 ring slots, one workgroup per tile
or persistent grids.  A configuration the planner declines (or that needs
more LDS than a workgroup has) is skipped and counted; the rest must match
the oracle bit for bit (exp: within one ulp; row sums of small integers:
exactly).  ACP_RANDOM_CASES sets the configurations per seed block (40 by
default; 2000 runs 24 000 configurations over the six entry points, and a
quarter as many persistent whole-line copies aimed at the blocked walk)."""
import os

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import async_copy_pipelining_amd as acp  # noqa: E402
from oracle import reference as REF  # noqa: E402
from tests.gpu_util import dev, empty_bytes, host, packed_strides, stream, ulp_diff  # noqa: E402

NP = {"u8": np.uint8, "u16": np.uint16, "u32": np.uint32, "f16": np.float16, "f32": np.float32}
BITS = {1: np.uint8, 2: np.uint16, 4: np.uint32}
SKIP = (acp.ACP_ERR_DECLINED, acp.ACP_ERR_UNSUPPORTED, acp.ACP_ERR_LDS)
CASES = int(os.environ.get("ACP_RANDOM_CASES", "40"))
SEED_BLOCKS = [0, max(1000, CASES)]   # two disjoint blocks of CASES seeds


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _shape(rng, dt, inner_choices=(64, 96, 128, 256, 320, 512, 1024)):
    r = int(rng.integers(2, 5))
    inner = int(rng.choice(inner_choices))
    shape = [int(rng.integers(1, 5)) for _ in range(r - 2)] + [int(rng.integers(1, 41)), inner]
    return tuple(shape)


def _box(rng, shape, esize):
    """Innermost box: the row or an even share of it (16-byte multiples);
    the next dim a power of two up to 16 (or the whole extent), outer dims
    1 or 2, so that most tiles split evenly over the workgroup's lanes."""
    box = []
    for d, e in enumerate(shape):
        if d == len(shape) - 1:
            cands = [b for b in (e, e // 2, e // 4, e // 8) if b > 0 and e % b == 0 and (b * esize) % 16 == 0]
            box.append(int(rng.choice(cands)))
        elif d == len(shape) - 2:
            box.append(min(e, int(rng.choice([1, 2, 4, 8, 16]))))
        else:
            box.append(min(e, int(rng.choice([1, 1, 2]))))
    return tuple(box)


def _threads(rng, tile_bytes, rounds16=False):
    """A workgroup size whose lanes split the tile evenly (at least 4 bytes
    each) in at most 8 rounds of 16 bytes; with rounds16, into 1, 2, 4 or 8
    whole 16-byte rounds (what the two-tensor, reduce-add and row-sum
    kernels take)."""
    if rounds16:
        ok = [t for t in (64, 128, 256, 512, 1024)
              if tile_bytes % (16 * t) == 0 and tile_bytes // (16 * t) in (1, 2, 4, 8)]
    else:
        ok = [t for t in (64, 128, 256, 512, 1024) if tile_bytes % (4 * t) == 0 and tile_bytes <= t * 16 * 8]
    return int(rng.choice(ok or [64]))


def _stage(rng, box):
    """A stage box dividing `box`: the innermost run whole, other dims divisors."""
    return tuple(_divisor(rng, b) for b in box[:-1]) + (box[-1],)


def _geometry(rng, dt, unit, inner_choices=(64, 96, 128, 256, 320, 512, 1024), whole_rows=False):
    """shape, box and stage with the stage a whole number of `unit` bytes (a
    wave's 64 lanes x 4 or 16 bytes), drawn again until one is (20 tries)."""
    es = np.dtype(NP[dt]).itemsize
    for _ in range(20):
        shape = _shape(rng, dt, inner_choices)
        box = _box(rng, shape, es)
        if whole_rows:
            box = box[:-1] + (shape[-1],)
        stage = _stage(rng, box)
        if (int(np.prod(stage)) * es) % unit == 0:
            break
    return shape, box, stage


def _divisor(rng, n):
    return int(rng.choice([k for k in range(1, n + 1) if n % k == 0]))


def _values(rng, dt, shape, kind="normal"):
    if dt in ("u8", "u16", "u32"):
        return rng.integers(0, np.iinfo(NP[dt]).max, size=shape, dtype=np.uint64).astype(NP[dt])
    if kind == "positive":
        return rng.uniform(0, 1e3, shape).astype(NP[dt])
    if kind == "exp":
        return rng.uniform(-8, 8, shape).astype(NP[dt])
    if kind == "ints":
        return rng.integers(-20, 21, size=shape).astype(NP[dt])
    if kind == "tiny":                                # float16 sums of up to 640 of these stay exact
        return rng.integers(-2, 3, size=shape).astype(NP[dt])
    return rng.standard_normal(shape).astype(NP[dt])


def _padded(rng, a):
    """Device copy of `a` whose innermost rows are padded by 0, 16 or 32
    bytes (filled with a sentinel); returns (buffer, strides)."""
    es = a.dtype.itemsize
    pad = int(rng.choice([0, 16, 32])) // es
    store = np.full(a.shape[:-1] + (a.shape[-1] + pad,), 0x7E if es == 1 else 0, dtype=a.dtype)
    if es > 1:
        store.view(BITS[es])[...] = {2: 0x7E5A, 4: 0x7FC0DEAD}[es]
    store[..., :a.shape[-1]] = a
    return dev(store), packed_strides(store.shape)


def _run(call):
    """Call an entry point; a declined, unsupported or LDS-bound configuration returns False."""
    try:
        call()
        return True
    except acp.AcpError as e:
        if e.status in SKIP:
            return False
        raise


def _check(op, got, want):
    if op == "exp":
        assert ulp_diff(got.reshape(-1), want.reshape(-1)).max() <= 1
    else:
        bits = BITS[got.dtype.itemsize]
        assert np.array_equal(got.view(bits), want.view(bits))


def _tally(ran, total, floor):
    say(f"{ran} of {total} configurations ran")
    assert ran >= floor, f"only {ran} of {total} random configurations ran"


@pytest.mark.parametrize("seed0", SEED_BLOCKS)
def test_random_tile_copy(seed0):
    ran = 0
    for seed in range(seed0, seed0 + CASES):
        rng = np.random.default_rng(seed)
        dt = str(rng.choice(["u8", "u16", "f16", "f32", "u32"]))
        es = np.dtype(NP[dt]).itemsize
        shape = _shape(rng, dt)
        if rng.random() < 0.2:                        # enough tiles for a persistent grid
            shape = (64,) + shape[1:]
        box, swz = _box(rng, shape, es), int(rng.integers(0, 4))
        threads = _threads(rng, int(np.prod(box)) * es)
        say(f"seed {seed}: tile_copy {dt} {shape} box {box} swizzle {swz} threads {threads}")
        x = _values(rng, dt, shape)
        xd, xs = _padded(rng, x)
        yd = empty_bytes(x.nbytes)
        try:
            src = acp.acp_encode_tiled(dt, xd, shape, xs, box, swz)
            dst = acp.acp_encode_tiled(dt, yd, shape, packed_strides(shape), box, swz)
        except acp.AcpError as e:
            assert e.status in SKIP
            continue
        if _run(lambda: acp.acp_tile_copy(src, dst, threads, stream())):
            ran += 1
            _check("copy", host(yd, NP[dt], shape), x)
    _tally(ran, CASES, CASES // 2)


@pytest.mark.parametrize("seed0", SEED_BLOCKS)
def test_random_blocked_walk_copies(seed0):
    # persistent copies whose staged rows are whole 128-byte lines walk
    # blocked runs of consecutive tiles: ragged tile counts, narrow tiles
    # staged in pairs, swizzles, line-aligned sources (non-temporal loads)
    # and padded ones (cached loads); most configurations must take that walk
    n_cases = max(8, CASES // 4)
    ran = blocked = 0
    for seed in range(seed0 + 50000, seed0 + 50000 + n_cases):
        rng = np.random.default_rng(seed)
        dt = str(rng.choice(["u8", "f16", "f32"]))
        es = np.dtype(NP[dt]).itemsize
        row_b = int(rng.choice([64, 128, 256]))          # tile row bytes (64: staged in pairs)
        cols = row_b // es
        inner = cols * int(rng.integers(2, 9))
        rows_box = int(rng.choice([8, 16, 32, 64]))
        n_rows = int(rng.integers(rows_box, 4 * rows_box + 1))
        per_slab = -(-n_rows // rows_box) * (inner // cols)
        shape = (-(-300 // per_slab) * 2 + int(rng.integers(0, 5)), n_rows, inner)
        box = (1, rows_box, cols)
        swz = int(rng.choice([0, 3])) if row_b <= 128 else 0
        threads = _threads(rng, rows_box * row_b)
        say(f"seed {seed}: blocked-walk copy {dt} {shape} box {box} swizzle {swz} threads {threads}")
        x = _values(rng, dt, shape)
        xd, xs = _padded(rng, x)
        yd = empty_bytes(x.nbytes)
        try:
            src = acp.acp_encode_tiled(dt, xd, shape, xs, box, swz)
            dst = acp.acp_encode_tiled(dt, yd, shape, packed_strides(shape), box, swz)
        except acp.AcpError as e:
            assert e.status in SKIP
            continue
        if _run(lambda: acp.acp_tile_copy(src, dst, threads, stream())):
            ran += 1
            blocked += acp.acp_last_kernel().endswith(" blocked-walk")
            _check("copy", host(yd, NP[dt], shape), x)
    _tally(ran, n_cases, n_cases // 2)
    assert blocked >= ran // 2, f"{blocked} of {ran} copies took the blocked walk"


@pytest.mark.parametrize("seed0", SEED_BLOCKS)
def test_random_tile_ewise(seed0):
    ran = 0
    for seed in range(seed0, seed0 + CASES):
        rng = np.random.default_rng(seed)
        op = str(rng.choice(["sqrt", "exp", "add", "mul", "fma", "zero"]))
        idt = str(rng.choice(["f16", "f32"]))
        odt = str(rng.choice(["f16", "f32"])) if op in ("sqrt", "exp") else idt
        n_in = {"sqrt": 1, "exp": 1, "add": 2, "mul": 2, "fma": 3, "zero": 1}[op]
        shape = _shape(rng, idt)
        if rng.random() < 0.3:
            shape = (int(rng.choice([64, 150])), 32, int(rng.choice([32, 64])))
        box = _box(rng, shape, 2)
        swz = int(rng.integers(0, 4))
        threads = _threads(rng, int(np.prod(box)) * np.dtype(NP[idt]).itemsize)
        say(f"seed {seed}: tile_ewise {op} {idt}->{odt} {shape} box {box} swizzle {swz} threads {threads}")
        kind = {"sqrt": "positive", "exp": "exp"}.get(op, "normal")
        ins = [_values(rng, idt, shape, kind) for _ in range(n_in)]
        st = packed_strides(shape)
        bufs = [dev(a) for a in ins]
        yd = empty_bytes(int(np.prod(shape)) * np.dtype(NP[odt]).itemsize)
        try:
            descs = [acp.acp_encode_tiled(idt, b, shape, st, box, swz) for b in bufs]
            out = acp.acp_encode_tiled(odt, yd, shape, st, box, swz)
        except acp.AcpError as e:
            assert e.status in SKIP
            continue
        if _run(lambda: acp.acp_tile_ewise(op, out, descs, threads, stream())):
            ran += 1
            _check(op, host(yd, NP[odt], shape), REF.ewise(op, ins, NP[odt]))
    _tally(ran, CASES, CASES // 2)


@pytest.mark.parametrize("seed0", SEED_BLOCKS)
def test_random_stream_ewise(seed0):
    ran = 0
    for seed in range(seed0, seed0 + CASES):
        rng = np.random.default_rng(seed)
        op = str(rng.choice(["sqrt", "exp", "zero", "fma", "add", "mul"]))
        row = op in ("fma", "add", "mul")
        idt = "f32" if row else str(rng.choice(["f16", "f32"]))
        odt = idt if op in ("zero",) or row else str(rng.choice(["f16", "f32"]))
        shape, box, stage = _geometry(rng, idt, 256)
        swz = int(rng.integers(0, 4))
        threads = _threads(rng, int(np.prod(stage)) * np.dtype(NP[idt]).itemsize)
        stages, wgs = int(rng.integers(2, 5)), int(rng.choice([0, 0, 3, 8]))
        say(f"seed {seed}: stream_ewise {op} {idt}->{odt} {shape} box {box} stage {stage} swizzle {swz} "
            f"threads {threads} S={stages} wg={wgs}")
        kind = {"sqrt": "positive", "exp": "exp"}.get(op, "normal")
        x = _values(rng, idt, shape, kind)
        xd, xs = _padded(rng, x)
        yd = empty_bytes(x.size * np.dtype(NP[odt]).itemsize)
        a = rng.uniform(-2, 2, shape[:-1]).astype(np.float32)
        b = rng.uniform(-2, 2, shape[:-1]).astype(np.float32)
        ad, bd = (dev(a), dev(b)) if row else (None, None)
        try:
            xdesc = acp.acp_encode_tiled(idt, xd, shape, xs, box, swz)
            ydesc = acp.acp_encode_tiled(odt, yd, shape, packed_strides(shape), box, swz)
        except acp.AcpError as e:
            assert e.status in SKIP
            continue
        if _run(lambda: acp.acp_stream_ewise(op, ydesc, xdesc, ad, bd, stage, stages, threads, wgs, stream())):
            ran += 1
            want = REF.stream_ewise(op, x, a if row else None, b if row else None, NP[odt])
            _check(op, host(yd, NP[odt], shape), want)
    _tally(ran, CASES, CASES // 2)


@pytest.mark.parametrize("seed0", SEED_BLOCKS)
def test_random_two_tensor_stream(seed0):
    ran = 0
    for seed in range(seed0, seed0 + CASES):
        rng = np.random.default_rng(seed)
        op, dt = str(rng.choice(["add", "mul"])), str(rng.choice(["f16", "f32"]))
        staging = str(rng.choice(["ring", "set"]))
        shape, box, stage = _geometry(rng, dt, 1024)
        swz = int(rng.integers(0, 4))
        threads = _threads(rng, int(np.prod(stage)) * np.dtype(NP[dt]).itemsize, rounds16=True)
        stages, wgs = int(rng.integers(2, 5)), int(rng.choice([0, 0, 3, 8]))
        say(f"seed {seed}: stream_binary {op} {dt} z={staging} {shape} box {box} stage {stage} swizzle {swz} "
            f"threads {threads} S={stages} wg={wgs}")
        x, z = _values(rng, dt, shape), _values(rng, dt, shape)
        st = packed_strides(shape)
        xd, zd = dev(x), dev(z)
        yd = empty_bytes(x.nbytes)
        try:
            xdesc, zdesc, ydesc = (acp.acp_encode_tiled(dt, t, shape, st, box, swz) for t in (xd, zd, yd))
        except acp.AcpError as e:
            assert e.status in SKIP
            continue
        if _run(lambda: acp.acp_stream_binary(op, ydesc, xdesc, zdesc, stage, stages, threads, wgs, staging,
                                              stream())):
            ran += 1
            _check(op, host(yd, NP[dt], shape), REF.ewise(op, [x, z], NP[dt]))
    _tally(ran, CASES, CASES // 2)


@pytest.mark.parametrize("seed0", SEED_BLOCKS)
def test_random_tile_reduce(seed0):
    ran = 0
    for seed in range(seed0, seed0 + CASES):
        rng = np.random.default_rng(seed)
        dt = str(rng.choice(["u32", "f32", "f16"]))
        es = np.dtype(NP[dt]).itemsize
        for _ in range(20):                           # tiles of whole 1 KiB wave blocks
            shape = _shape(rng, dt)
            box = list(_box(rng, shape, es))
            dshape = list(shape)
            for d in range(len(shape) - 1):           # sum over some dims whose box is 1
                if rng.random() < 0.4:
                    box[d], dshape[d] = 1, 1
            if (int(np.prod(box)) * es) % 1024 == 0:
                break
        box, dshape = tuple(box), tuple(dshape)
        swz = int(rng.integers(0, 4))
        threads = _threads(rng, int(np.prod(box)) * np.dtype(NP[dt]).itemsize, rounds16=True)
        say(f"seed {seed}: tile_reduce {dt} {shape} -> {dshape} box {box} swizzle {swz} threads {threads}")
        # every partial sum exactly representable: the result is order-free
        kind = {"u32": "normal", "f32": "ints", "f16": "tiny"}[dt]
        src, dst = _values(rng, dt, shape, kind), _values(rng, dt, dshape, kind)
        sd, dd = dev(src), dev(dst)
        try:
            sdesc = acp.acp_encode_tiled(dt, sd, shape, packed_strides(shape), box, swz)
            ddesc = acp.acp_encode_tiled(dt, dd, dshape, packed_strides(dshape), box)
        except acp.AcpError as e:
            assert e.status in SKIP
            continue
        if _run(lambda: acp.acp_tile_reduce("add", ddesc, sdesc, threads, stream())):
            ran += 1
            _check("add", host(dd, NP[dt], dshape), REF.tile_reduce_add(dst, src))
    _tally(ran, CASES, CASES // 2)


@pytest.mark.parametrize("seed0", SEED_BLOCKS)
def test_random_row_reduction(seed0):
    ran = 0
    for seed in range(seed0, seed0 + CASES):
        rng = np.random.default_rng(seed)
        dt = str(rng.choice(["f16", "f32"]))
        shape, box, stage = _geometry(rng, dt, 1024, (64, 128, 256, 512, 1024, 2048), whole_rows=True)
        swz = int(rng.integers(0, 4))
        threads = _threads(rng, int(np.prod(stage)) * np.dtype(NP[dt]).itemsize, rounds16=True)
        stages, wgs = int(rng.integers(2, 5)), int(rng.choice([0, 0, 3, 8]))
        say(f"seed {seed}: reduce_rows {dt} {shape} box {box} stage {stage} swizzle {swz} threads {threads} "
            f"S={stages} wg={wgs}")
        x = _values(rng, dt, shape, "ints")
        xd, xs = _padded(rng, x)
        rows = int(np.prod(shape[:-1]))
        yd = empty_bytes(rows * 4 + 64)
        try:
            xdesc = acp.acp_encode_tiled(dt, xd, shape, xs, box, swz)
        except acp.AcpError as e:
            assert e.status in SKIP
            continue
        if _run(lambda: acp.acp_stream_reduce_rows("add", yd, xdesc, stage, stages, threads, wgs, stream())):
            ran += 1
            y = host(yd, np.float32)
            assert np.all(y.view(np.uint8)[rows * 4:] == 0xA5)
            assert np.array_equal(y[:rows].reshape(shape[:-1]), REF.reduce_rows(x))
    _tally(ran, CASES, CASES // 2)
