"""CPU-side checks of the C-ABI library: it loads, exports every entry point
the header declares, and its host planner agrees field by field with the
oracle planner (no GPU work is launched here)."""
import os
import random
import re

import pytest

import async_copy_pipelining_amd as acp
from oracle import plan as P

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE_BASE = 1 << 20   # encode never dereferences the address


def test_library_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "acp.h")) as f:
        header = f.read()
    declared = set(re.findall(r"^\s*(?:acp_status|int|const char\*)\s+(acp_\w+)\s*\(", header, re.M))
    assert declared == set(acp.EXPORTED)
    for name in declared:
        assert hasattr(acp._lib, name)
    assert acp.acp_abi_version() == 1


# kernel limits of the library (not rules of the pages): loads per tile and
# LDS-image axes its kernels index; beyond them it answers UNSUPPORTED
LIB_MAX_ISSUES = 256
LIB_MAX_IMAGE_AXES = 12


class _Unsupported(Exception):
    pass


def _cmp(dt, shape, strides, box, swz, threads, copy_only, base=FAKE_BASE):
    """Run both planners; return (oracle outcome, library outcome)."""
    try:
        p = P.plan_box(P.ESIZE[dt], shape, strides, box, swz, copy_only, base)
        if p.issues > LIB_MAX_ISSUES or len(p.image_axes) > LIB_MAX_IMAGE_AXES:
            # a legal plan beyond what the library's kernels index
            raise _Unsupported()
        if threads:
            P.partition(p, threads, base_addr=base)
        o = ("ok", p.rank, [d.extent for d in reversed(p.dims)], [d.stride for d in reversed(p.dims)],
             [d.box for d in reversed(p.dims)], p.issues, len(p.image_axes), p.promoted,
             p.vec, p.vec_bytes, p.outer, p.tile_bytes)
    except P.Declined:
        o = ("declined",)
    except P.Invalid:
        o = ("invalid",)
    except _Unsupported:
        o = ("unsupported",)
    try:
        # encode checks the box with promotion allowed; the query then plans
        # with the requested mode and thread count
        d = acp.acp_encode_tiled(dt, base, shape, strides, box, swz)
        q = acp.acp_plan_query(d, threads, copy_only)
        c = ("ok", q["rank"], q["dims"], q["strides"], q["box"], q["issues"], q["n_image_axes"], q["promoted"],
             q["vec"], q["vec_bytes"], q["outer"], q["tile_bytes"])
    except acp.AcpError as e:
        c = {acp.ACP_ERR_DECLINED: ("declined",), acp.ACP_ERR_INVALID: ("invalid",),
             acp.ACP_ERR_UNSUPPORTED: ("unsupported",)}[e.status]
    return o, c


WORKED = [
    ("f16", (8, 256), (256, 1), (8, 256), 3, 64, True),
    ("f32", (65536, 32, 32), (1024, 32, 1), (1, 32, 32), 0, 256, False),
    ("f16", (128, 500, 1024), (512000, 1024, 1), (1, 128, 32), 0, 128, True),
    ("f32", (128, 500, 1024), (512000, 1024, 1), (1, 4, 1024), 0, 256, False),
    ("f16", (4, 8, 64, 128, 256), (17301504, 2162688, 33792, 264, 1), (1, 1, 1, 64, 64), 3, 256, False),
    ("f16", (4, 8, 64, 128, 256), (17301504, 2162688, 33792, 264, 1), (1, 2, 16, 64, 64), 3, 256, False),
    ("u8", (8, 128), (128, 1), (8, 128), 0, 64, True),
    ("f16", (600, 64), (64, 1), (600, 64), 0, 128, False),
]


@pytest.mark.parametrize("case", WORKED, ids=[str(i) for i in range(len(WORKED))])
def test_planner_matches_oracle_on_worked_cases(case):
    o, c = _cmp(*case)
    assert o[0] == "ok" and o == c


def test_planner_matches_oracle_on_alignment_table():
    for base, vb, outer in ((FAKE_BASE, 16, 4), (FAKE_BASE + 8, 4, 16), (FAKE_BASE + 4, 4, 16)):
        o, c = _cmp("f16", (128, 32), (32, 1), (128, 32), 0, 128, True, base=base)
        assert o == c and c[9] == vb and c[10] == outer
    o, c = _cmp("f16", (128, 32), (32, 1), (128, 32), 0, 128, True, base=FAKE_BASE + 2)
    assert o == c == ("declined",)


def test_planner_matches_oracle_randomized():
    rng = random.Random(2024)
    n_ok = n_decl = 0
    for _ in range(1500):
        r = rng.randint(1, 7)
        dt = rng.choice(["u8", "u16", "f16", "f32", "u64"])
        shape = [rng.choice([1, 2, 3, 4, 5, 8, 16, 33]) for _ in range(r)]
        shape[-1] = rng.choice([4, 8, 16, 24, 32, 64, 96, 128, 256, 300, 512, 1024, 2048])
        box = [rng.randint(1, s) for s in shape]
        if rng.random() < 0.7:
            box[-1] = rng.choice([b for b in range(1, shape[-1] + 1) if shape[-1] % b == 0])
        strides, st = [], 1
        pad = rng.choice([0, 0, 0, 2, 8, 16])
        for k, ext in enumerate(reversed(shape)):
            strides.append(st)
            st *= ext + (pad if k == 0 else 0)
        strides = list(reversed(strides))
        if rng.random() < 0.03:
            strides[-1] = 2
        swz = rng.choice([0, 1, 2, 3])
        threads = rng.choice([0, 64, 128, 256, 1024])
        copy_only = rng.random() < 0.5
        base = FAKE_BASE + rng.choice([0, 0, 0, 4, 8])
        o, c = _cmp(dt, shape, strides, box, swz, threads, copy_only, base)
        assert o == c, (dt, shape, strides, box, swz, threads, copy_only, base)
        n_ok += o[0] == "ok"
        n_decl += o[0] == "declined"
    assert n_ok > 300 and n_decl > 50


def test_status_codes_and_reasons():
    with pytest.raises(acp.AcpError) as e:
        acp.acp_encode_tiled("f16", FAKE_BASE, (8, 256), (1, 8), (8, 256))
    assert e.value.status == acp.ACP_ERR_DECLINED and "innermost stride" in e.value.reason
    with pytest.raises(acp.AcpError) as e:
        acp.acp_encode_tiled("f16", 0, (8, 256), (256, 1), (8, 256))
    assert e.value.status == acp.ACP_ERR_INVALID
    with pytest.raises(acp.AcpError) as e:
        acp.acp_encode_tiled("f16", FAKE_BASE, (8, 12), (12, 1), (8, 12), acp.ACP_SWIZZLE_128B)
    assert e.value.status == acp.ACP_ERR_DECLINED and "16-byte" in e.value.reason
    # a 192-byte inner box under the 128-byte swizzle is shrunk into two loads
    d = acp.acp_encode_tiled("f16", FAKE_BASE, (8, 96), (96, 1), (8, 96), acp.ACP_SWIZZLE_128B)
    assert acp.acp_plan_query(d, 64)["issues"] == 2
    # legal, but deeper than the kernels index: unsupported, not declined
    shape = (7, 7, 7, 7, 7, 7, 7, 64)
    strides, st = [], 1
    for ext in reversed(shape):
        strides.append(st)
        st *= ext + 1
    with pytest.raises(acp.AcpError) as e:
        acp.acp_encode_tiled("f32", FAKE_BASE, shape, tuple(reversed(strides)), shape)
    assert e.value.status == acp.ACP_ERR_UNSUPPORTED and "kernel limits" in e.value.reason
    d = acp.acp_encode_tiled("f16", FAKE_BASE, (8, 256), (256, 1), (8, 256))
    with pytest.raises(acp.AcpError) as e:
        acp.acp_plan_query(d, 96)
    assert e.value.status == acp.ACP_ERR_INVALID
    # stream_ewise argument errors are caught on the host before any launch
    x = acp.acp_encode_tiled("f32", FAKE_BASE, (4, 8, 256), (2048, 256, 1), (1, 4, 256))
    y = acp.acp_encode_tiled("f32", FAKE_BASE * 2, (4, 8, 256), (2048, 256, 1), (1, 4, 256))
    with pytest.raises(acp.AcpError) as e:
        acp.acp_stream_ewise("fma", y, x, FAKE_BASE * 3, FAKE_BASE * 4, (1, 4, 256), 5, 256)
    assert e.value.status == acp.ACP_ERR_INVALID and "stages" in e.value.reason
    with pytest.raises(acp.AcpError) as e:
        acp.acp_stream_ewise("fma", y, x, None, FAKE_BASE * 4, (1, 4, 256), 3, 256)
    assert e.value.status == acp.ACP_ERR_INVALID
    with pytest.raises(acp.AcpError) as e:
        acp.acp_stream_ewise("fma", y, x, FAKE_BASE * 3, FAKE_BASE * 4, (1, 3, 256), 3, 256)
    assert e.value.status == acp.ACP_ERR_INVALID and "divide" in e.value.reason
    with pytest.raises(acp.AcpError) as e:
        acp.acp_tile_copy(x, acp.acp_encode_tiled("f16", FAKE_BASE, (4, 8, 256), (2048, 256, 1), (1, 4, 256)), 256)
    assert e.value.status == acp.ACP_ERR_INVALID and "valid copy" in e.value.reason
    assert acp.acp_last_error() != ""
    # reduce-add shape and dtype rules are checked on the host
    src = acp.acp_encode_tiled("f32", FAKE_BASE, (4, 8, 256), (2048, 256, 1), (1, 4, 256))
    for dshape, dbox, dt, why in (((2, 8, 256), (1, 4, 256), "f32", "equal the source"),
                                  ((1, 8, 256), (1, 8, 256), "f32", "boxes differ"),
                                  ((1, 8, 256), (1, 4, 256), "u32", "dtypes differ")):
        d = acp.acp_encode_tiled(dt, FAKE_BASE * 5, dshape, (2048, 256, 1), dbox)
        with pytest.raises(acp.AcpError) as e:
            acp.acp_tile_reduce("add", d, src, 256)
        assert e.value.status == acp.ACP_ERR_INVALID and why in e.value.reason
    with pytest.raises(acp.AcpError) as e:
        acp.acp_tile_reduce("mul", src, src, 256)
    assert e.value.status == acp.ACP_ERR_INVALID
    # the reference stream copy checks its arguments before any launch
    for dst, src, n, why in ((FAKE_BASE, FAKE_BASE + 64, 128, "overlap"), (FAKE_BASE, FAKE_BASE * 8, 100, "16-byte"),
                             (FAKE_BASE, FAKE_BASE * 8, -16, "bad"), (None, FAKE_BASE, 16, "bad")):
        with pytest.raises(acp.AcpError) as e:
            acp.acp_debug_stream_copy(dst, src, n)
        assert e.value.status == acp.ACP_ERR_INVALID and why in e.value.reason


def test_reference_copy_arguments_are_checked_on_the_host():
    # the copy-shape and tiled-copy references refuse bad requests before
    # any launch: unbuilt shapes are unsupported, malformed ones invalid
    for args, status, why in (
            ((256, 3, 1, 1), acp.ACP_ERR_UNSUPPORTED, "shape"),
            ((96, 4, 1, 1), acp.ACP_ERR_UNSUPPORTED, "shape"),
            ((256, 4, 2, 1), acp.ACP_ERR_INVALID, "policies"),
            ((256, 4, 1, -1), acp.ACP_ERR_INVALID, "policies")):
        with pytest.raises(acp.AcpError) as e:
            acp.acp_debug_stream_copy_shape(FAKE_BASE * 8, FAKE_BASE, 4096, 0, *args)
        assert e.value.status == status and why in e.value.reason, e.value.reason
    with pytest.raises(acp.AcpError) as e:
        acp.acp_debug_stream_copy_shape(FAKE_BASE, FAKE_BASE + 64, 4096, 0, 256, 4, 1, 1)
    assert e.value.status == acp.ACP_ERR_INVALID and "overlap" in e.value.reason
    shape, strides = (2, 300, 352), (300 * 352, 352, 1)
    out = FAKE_BASE * 64
    for kw, why in (
            (dict(esize=3), "element size"),
            (dict(threads=64), "threads"),
            (dict(tiles_per_trip=3), "tiles per trip"),
            (dict(box=(2, 128, 32)), "dim 0"),
            (dict(box=(1, 128, 3)), "16-byte"),
            (dict(box=(1, 256, 32)), "8 chunks"),
            (dict(strides=(300 * 352, 352, 2)), "innermost"),
            (dict(strides=(300 * 352, 348, 1)), "16-byte multiples"),
            (dict(src=FAKE_BASE + 2), "aligned"),
            (dict(dst=FAKE_BASE + 4096), "overlap")):
        a = dict(dst=out, src=FAKE_BASE, esize=2, shape=shape, strides=strides, box=(1, 128, 32),
                 tiles_per_trip=2, threads=128)
        a.update(kw)
        with pytest.raises(acp.AcpError) as e:
            acp.acp_debug_copy_tiles(a["dst"], a["src"], a["esize"], a["shape"], a["strides"], a["box"],
                                     a["tiles_per_trip"], a["threads"])
        assert e.value.status == acp.ACP_ERR_INVALID and why in e.value.reason, (kw, e.value.reason)


def test_memory_shared_between_a_written_tensor_and_another_operand_is_rejected():
    """Workgroups read and write different tensors with no ordering between
    them, so every entry point refuses a written tensor that shares bytes
    with another operand (checked on the host, before any launch)."""
    shape, strides, box = (4, 8, 256), (2048, 256, 1), (1, 4, 256)
    span = 4 * 8 * 256 * 4
    x = acp.acp_encode_tiled("f32", FAKE_BASE, shape, strides, box)
    near = acp.acp_encode_tiled("f32", FAKE_BASE + span - 16, shape, strides, box)   # last 16 bytes shared
    far = acp.acp_encode_tiled("f32", FAKE_BASE + span, shape, strides, box)         # adjacent, disjoint
    cases = [
        (lambda: acp.acp_tile_copy(x, near, 256), "share memory"),
        (lambda: acp.acp_tile_copy(x, x, 256), "share memory"),
        (lambda: acp.acp_tile_ewise("sqrt", near, [x], 256), "shares memory"),
        (lambda: acp.acp_stream_ewise("exp", near, x, None, None, box, 2, 256), "share memory"),
        (lambda: acp.acp_stream_ewise("exp", x, x, None, None, box, 2, 256), "share memory"),
        (lambda: acp.acp_stream_ewise("fma", far, x, FAKE_BASE + span + 64, FAKE_BASE * 8, box, 2, 256),
         "per-row scalar"),
        (lambda: acp.acp_stream_binary("add", near, far, far, box, 2, 256), "shares memory"),
        (lambda: acp.acp_stream_binary("add", far, x, near, box, 2, 256), "shares memory"),
        (lambda: acp.acp_tile_reduce("add", near, x, 256), "share memory"),
        (lambda: acp.acp_stream_reduce_rows("add", FAKE_BASE + 64, x, (1, 4, 256), 2, 256), "shares memory"),
        (lambda: acp.acp_stream_reduce_rows("add", FAKE_BASE * 8 + 2, x, (1, 4, 256), 2, 256), "aligned"),
    ]
    for call, why in cases:
        with pytest.raises(acp.AcpError) as e:
            call()
        assert e.value.status == acp.ACP_ERR_INVALID and why in e.value.reason, e.value.reason
    # a float16 output over the bytes of a float32 operand: the same base,
    # but not element for element, so refused as well
    h = acp.acp_encode_tiled("f16", FAKE_BASE, shape, strides, box)
    with pytest.raises(acp.AcpError) as e:
        acp.acp_tile_ewise("sqrt", h, [x], 256)
    assert e.value.status == acp.ACP_ERR_INVALID


def test_host_calls_from_many_threads():
    # encode and plan from eight threads at once: every answer, and every
    # rejection reason (kept per thread), equals the single-threaded one
    import threading
    cases = [c[:7] for c in WORKED] + [
        ("f16", (8, 256), (256, 1), (8, 300), 0, 64, True),           # declined: no vector width fits
        ("f32", (64, 30), (30, 1), (4, 30), 3, 64, False),            # declined: row not in 16-byte chunks
        ("f16", (8, 256), (256, 2), (8, 256), 0, 64, True),           # declined: innermost stride not 1
        ("f32", (600, 64), (64, 1), (600, 64), 0, 96, False),         # invalid: threads not a multiple of 64
    ]

    def run(case):
        dt, shape, strides, box, swz, threads, copy_only = case
        try:
            d = acp.acp_encode_tiled(dt, FAKE_BASE, shape, strides, box, swz)
            q = acp.acp_plan_query(d, threads, copy_only)
            return ("ok", tuple(sorted((k, str(v)) for k, v in q.items())))
        except acp.AcpError as e:
            return ("err", e.status, str(e))

    want = [run(c) for c in cases]
    assert any(w[0] == "err" for w in want) and any(w[0] == "ok" for w in want)
    errors = []
    start = threading.Barrier(8)

    def worker(k):
        order = list(range(len(cases)))
        random.Random(k).shuffle(order)
        start.wait()
        for _ in range(200):
            for i in order:
                got = run(cases[i])
                if got != want[i]:
                    errors.append((k, i, got, want[i]))
                    return

    threads = [threading.Thread(target=worker, args=(k,)) for k in range(8)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    assert not errors, errors[:3]
