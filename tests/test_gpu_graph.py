"""The pipelined entry points inside a captured HIP graph: each call
enqueues plain kernel launches on the caller's stream (no allocation, no
memset), so a graph captured on that stream replays them.  Every replay,
with eager work and synchronization between replays, must equal the
oracle."""
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
