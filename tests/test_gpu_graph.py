"""The pipelined entry points inside a captured HIP graph: each call
enqueues plain kernel launches on the caller's stream (no allocation, no
memset), so a graph captured on that stream replays them.  Every replay,
with eager work and synchronization between replays, must equal the
oracle (a reduce-add's destination is restored before each replay, since
the call accumulates into it)."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import async_copy_pipelining_amd as acp  # noqa: E402
import workloads as W  # noqa: E402
from oracle import reference as REF  # noqa: E402
from tests.gpu_util import dev, empty_bytes, encode, host, packed_strides  # noqa: E402


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def test_graph_replays_stream_fma_tile_sqrt_and_row_sums():
    say("graph capture: streamed fma, tile sqrt, row sums; three replays")
    shape, stage = (4, 37, 1024), (1, 4, 1024)
    x, a, b = W.fma_rows_f32(shape, seed=9)
    xd, ad, bd = dev(x), dev(a), dev(b)
    yd = empty_bytes(x.nbytes)
    st = packed_strides(shape)
    xdesc, ydesc = encode("f32", xd, shape, st, stage), encode("f32", yd, shape, st, stage)
    t = np.abs(W.sqrt_tiles_f32(600, seed=10))
    td, ud = dev(t), empty_bytes(t.nbytes)
    tdesc = encode("f32", td, t.shape, packed_strides(t.shape), (1, 32, 32))
    udesc = encode("f32", ud, t.shape, packed_strides(t.shape), (1, 32, 32))
    rows = 4 * 37
    rd = empty_bytes(rows * 4)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        h = torch.cuda.current_stream().cuda_stream
        acp.acp_stream_ewise("fma", ydesc, xdesc, ad, bd, stage, 4, 256, 8, h)
        acp.acp_tile_ewise("sqrt", udesc, [tdesc], 256, h)
        acp.acp_stream_reduce_rows("add", rd, xdesc, stage, 2, 256, 8, h)
    want_y = REF.stream_ewise("fma", x, a, b, np.float32).view(np.uint32)
    want_u = REF.ewise("sqrt", [t], np.float32).view(np.uint32)
    for replay in range(3):
        yd.fill_(0xA5)
        ud.fill_(0xA5)
        rd.fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(yd, np.float32, shape).view(np.uint32), want_y), replay
        assert np.array_equal(host(ud, np.float32, t.shape).view(np.uint32), want_u), replay
        got = host(rd, np.float32, shape[:-1])
        bound = REF.recursive_sum_bound(x, shape[-1] - 1) + np.spacing(np.abs(REF.reduce_rows(x)))
        assert np.all(np.abs(got.astype(np.float64) - REF.reduce_rows(x)) <= bound), replay


def test_graph_replays_copy_reduce_add_and_two_tensor_streams():
    say("graph capture: swizzled tile copy, reduce-add over a batch dim, two-tensor streams (ring and Set)")
    # seven swizzled 8x256 float16 tiles
    c = W.tile_bits_f16((7, 8, 256), seed=1)
    cd, co = dev(c), empty_bytes(c.nbytes)
    csrc = encode("f16", cd, (7, 8, 256), (2048, 256, 1), (1, 8, 256), acp.ACP_SWIZZLE_128B)
    cdst = encode("f16", co, (7, 8, 256), (2048, 256, 1), (1, 8, 256), acp.ACP_SWIZZLE_128B)
    # reduce-add of 8 slabs into one, on small integers (every partial sum exact)
    rng = np.random.default_rng(52)
    src = rng.integers(-50, 51, size=(8, 64, 256)).astype(np.float32)
    dst0 = rng.integers(-50, 51, size=(1, 64, 256)).astype(np.float32)
    sd, dd0 = dev(src), dev(dst0)
    dd = dd0.clone()
    sdesc = encode("f32", sd, src.shape, packed_strides(src.shape), (1, 16, 256))
    ddesc = encode("f32", dd, dst0.shape, packed_strides(dst0.shape), (1, 16, 256))
    # x + z (z on the ring) and x * z (z staged "Set")
    shape, box = (3, 36, 1024), (1, 4, 1024)
    x = rng.standard_normal(shape).astype(np.float32)
    z = rng.standard_normal(shape).astype(np.float32)
    xd, zd, yad, ymd = dev(x), dev(z), empty_bytes(x.nbytes), empty_bytes(x.nbytes)
    st = packed_strides(shape)
    xdesc, zdesc = encode("f32", xd, shape, st, box), encode("f32", zd, shape, st, box)
    yadesc, ymdesc = encode("f32", yad, shape, st, box), encode("f32", ymd, shape, st, box)
    s = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=s):
        h = torch.cuda.current_stream().cuda_stream
        acp.acp_tile_copy(csrc, cdst, 64, h)
        acp.acp_tile_reduce("add", ddesc, sdesc, 256, h)
        acp.acp_stream_binary("add", yadesc, xdesc, zdesc, box, 3, 256, 5, "ring", h)
        acp.acp_stream_binary("mul", ymdesc, xdesc, zdesc, box, 3, 256, 5, "set", h)
    want_c = c.view(np.uint16).reshape(-1)
    want_d = REF.tile_reduce_add(dst0, src).view(np.uint32)
    want_a = REF.ewise("add", [x, z], np.float32).view(np.uint32)
    want_m = REF.ewise("mul", [x, z], np.float32).view(np.uint32)
    for replay in range(3):
        co.fill_(0xA5)
        yad.fill_(0xA5)
        ymd.fill_(0xA5)
        dd.copy_(dd0)                  # the reduce-add accumulates into its destination
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host(co, np.uint16), want_c), replay
        assert np.array_equal(host(dd, np.float32, dst0.shape).view(np.uint32), want_d), replay
        assert np.array_equal(host(yad, np.float32, shape).view(np.uint32), want_a), replay
        assert np.array_equal(host(ymd, np.float32, shape).view(np.uint32), want_m), replay
