"""The entry points called from several host threads at once, each on its
own stream.  The library keeps its prepared launches, its last-kernel name
and its error reason per thread, its device attributes in atomics, and
raises a kernel's dynamic-LDS limit (process state) only upward under a
lock, so concurrent callers neither see each other's state nor race on it:
every thread's results must equal the oracle and every thread must see its
own kernel names.  Two threads run the same streamed-fma kernel, one with
4 slots (128 KiB of LDS) and 2 slots in turn, the other with 2 slots
only, so a smaller launch on one thread must not lower the limit the other
relies on."""
import threading

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import async_copy_pipelining_amd as acp  # noqa: E402
import workloads as W  # noqa: E402
from oracle import reference as REF  # noqa: E402
from tests.gpu_util import dev, empty_bytes, encode, host, packed_strides  # noqa: E402

ROUNDS = 25


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def test_entry_points_from_five_threads_on_their_own_streams():
    say(f"five host threads, one stream each, {ROUNDS} rounds of two calls per thread")
    # streamed fma with 32 KiB stages, alternating 4 slots (128 KiB of LDS)
    # and 2 slots (64 KiB): two prepared launches of one kernel per thread
    shape, stage = (4, 40, 1024), (1, 8, 1024)
    x, a, b = W.fma_rows_f32(shape, seed=9)
    xd, ad, bd = dev(x), dev(a), dev(b)
    y0, y0b, y0c = empty_bytes(x.nbytes), empty_bytes(x.nbytes), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    xdesc = encode("f32", xd, shape, st, stage)
    y0desc, y0bdesc = encode("f32", y0, shape, st, stage), encode("f32", y0b, shape, st, stage)
    y0cdesc = encode("f32", y0c, shape, st, stage)
    # tile sqrt, at 256 and 128 threads
    t = np.abs(W.sqrt_tiles_f32(600, seed=10))
    td, u1, u1b = dev(t), empty_bytes(t.nbytes), empty_bytes(t.nbytes)
    tst = packed_strides(t.shape)
    tdesc = encode("f32", td, t.shape, tst, (1, 32, 32))
    u1desc, u1bdesc = encode("f32", u1, t.shape, tst, (1, 32, 32)), encode("f32", u1b, t.shape, tst, (1, 32, 32))
    # swizzled 8x256 f16 tiles: one tile, and a grid of seven
    c = W.tile_bits_f16((7, 8, 256), seed=1)
    cd, c2, c2b = dev(c), empty_bytes(c.nbytes), empty_bytes(c.nbytes)
    one_src = encode("f16", cd, (8, 256), (256, 1), (8, 256), acp.ACP_SWIZZLE_128B)
    one_dst = encode("f16", c2b, (8, 256), (256, 1), (8, 256), acp.ACP_SWIZZLE_128B)
    grid_src = encode("f16", cd, (7, 8, 256), (2048, 256, 1), (1, 8, 256), acp.ACP_SWIZZLE_128B)
    grid_dst = encode("f16", c2, (7, 8, 256), (2048, 256, 1), (1, 8, 256), acp.ACP_SWIZZLE_128B)
    # row sums at 2 and 3 slots, stage (1,4,1024)
    r3, r3b = empty_bytes(4 * 40 * 4), empty_bytes(4 * 40 * 4)

    def fma(h, i):
        if i % 2:
            acp.acp_stream_ewise("fma", y0desc, xdesc, ad, bd, stage, 4, 256, 8, h)
        else:
            acp.acp_stream_ewise("fma", y0bdesc, xdesc, ad, bd, stage, 2, 256, 8, h)
        return "stream linear grid"

    def fma_small(h, i):
        acp.acp_stream_ewise("fma", y0cdesc, xdesc, ad, bd, stage, 2, 256, 8, h)
        return "stream linear grid"

    def sqrt(h, i):
        if i % 2:
            acp.acp_tile_ewise("sqrt", u1desc, [tdesc], 256, h)
        else:
            acp.acp_tile_ewise("sqrt", u1bdesc, [tdesc], 128, h)
        return "tile linear grid"

    def copy(h, i):
        if i % 2:
            acp.acp_tile_copy(grid_src, grid_dst, 64, h)
        else:
            acp.acp_tile_copy(one_src, one_dst, 64, h)
        return "copy linear grid"

    def rows(h, i):
        acp.acp_stream_reduce_rows("add", r3 if i % 2 else r3b, xdesc, (1, 4, 1024), 2 + i % 2, 256, 8, h)
        return "row reduction"

    fns = (fma, sqrt, copy, rows, fma_small)
    streams = [torch.cuda.Stream() for _ in fns]
    errors, seen = [], [set() for _ in fns]
    start = threading.Barrier(len(fns))

    def worker(k, fn):
        try:
            h = streams[k].cuda_stream
            start.wait()
            for i in range(ROUNDS):
                want = fn(h, i)
                got = acp.acp_last_kernel()
                seen[k].add(got)
                if want not in got:
                    errors.append(f"thread {k}: last kernel {got!r}, expected {want!r}")
                # a rejected call sets this thread's reason only
                try:
                    acp.acp_tile_copy(one_src, one_src, 64, h)
                except acp.AcpError as e:
                    if "share memory" not in str(e):
                        errors.append(f"thread {k}: reason {e}")
                else:
                    errors.append(f"thread {k}: overlapping copy accepted")
        except Exception as e:  # pragma: no cover - reported below
            errors.append(f"thread {k}: {type(e).__name__}: {e}")

    threads = [threading.Thread(target=worker, args=(k, fn)) for k, fn in enumerate(fns)]
    for th in threads:
        th.start()
    for th in threads:
        th.join()
    torch.cuda.synchronize()
    assert not errors, errors[:5]
    assert all(len(s) >= 2 for s in seen[:3]), seen   # both launches of each thread ran
    want_y = REF.stream_ewise("fma", x, a, b, np.float32).view(np.uint32)
    assert np.array_equal(host(y0, np.float32, shape).view(np.uint32), want_y)
    assert np.array_equal(host(y0b, np.float32, shape).view(np.uint32), want_y)
    assert np.array_equal(host(y0c, np.float32, shape).view(np.uint32), want_y)
    want_u = REF.ewise("sqrt", [t], np.float32).view(np.uint32)
    assert np.array_equal(host(u1, np.float32, t.shape).view(np.uint32), want_u)
    assert np.array_equal(host(u1b, np.float32, t.shape).view(np.uint32), want_u)
    assert np.array_equal(host(c2, np.uint16), c.view(np.uint16).reshape(-1))
    one = host(c2b, np.uint16)
    assert np.array_equal(one[:2048], c.view(np.uint16).reshape(-1)[:2048]) and np.all(one[2048:] == 0xA5A5)
    exact = REF.reduce_rows(x)
    bound = REF.recursive_sum_bound(x, shape[-1] - 1) + np.spacing(np.abs(exact))
    for r in (r3, r3b):
        got = host(r, np.float32, shape[:-1]).astype(np.float64)
        assert np.all(np.abs(got - exact) <= bound)
