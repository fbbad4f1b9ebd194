"""Child process of test_gpu_env.py: runs the linear-grid kernels under the
environment the parent sets (the library reads its knobs once per process)
and checks each result against the oracle.  Prints one line per case and
"all ok" at the end; any mismatch raises."""
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import torch  # noqa: E402

import async_copy_pipelining_amd as acp  # noqa: E402
import workloads as W  # noqa: E402
from oracle import reference as REF  # noqa: E402
from tests.gpu_util import dev, empty_bytes, encode, host, packed_strides, stream  # noqa: E402


def say(msg):
    print(msg, flush=True)


def expect_kind(prefix):
    kind = acp.acp_last_kernel()
    if not kind.startswith(prefix):
        raise AssertionError(f"expected a '{prefix}' launch, got '{kind}'")
    return kind


def fma_stream():
    shape, stage = (3, 36, 1024), (1, 4, 1024)     # 27 stages on a linear grid
    x, a, b = W.fma_rows_f32(shape, seed=11)
    xd, ad, bd = dev(x), dev(a), dev(b)
    yd = empty_bytes(x.nbytes)
    st = packed_strides(shape)
    for stages in (2, 3, 4):
        acp.acp_stream_ewise("fma", encode("f32", yd, shape, st, stage), encode("f32", xd, shape, st, stage),
                             ad, bd, stage, stages, 256, 5, stream())
        kind = expect_kind("stream linear grid")
        y = host(yd, np.float32, shape)
        ref = REF.stream_ewise("fma", x, a, b, np.float32)
        assert np.array_equal(y.view(np.uint32), ref.view(np.uint32)), ("fma", stages)
        say(f"fma stream S={stages}: {kind}")


def binary_stream():
    shape, stage = (3, 36, 1024), (1, 4, 1024)
    rng = np.random.default_rng(12)
    x = rng.standard_normal(shape, dtype=np.float32)
    z = rng.standard_normal(shape, dtype=np.float32)
    xd, zd = dev(x), dev(z)
    yd = empty_bytes(x.nbytes)
    st = packed_strides(shape)
    acp.acp_stream_binary("add", encode("f32", yd, shape, st, stage), encode("f32", xd, shape, st, stage),
                          encode("f32", zd, shape, st, stage), stage, 2, 256, 7, "ring", stream())
    kind = expect_kind("stream linear grid")
    y = host(yd, np.float32, shape)
    ref = REF.ewise("add", [x, z], np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32)), "add"
    say(f"two-tensor add: {kind}")


def row_sums():
    shape, stage = (3, 36, 1024), (1, 4, 1024)
    rng = np.random.default_rng(13)
    x = rng.integers(-50, 51, size=shape).astype(np.float32)   # every partial sum exact
    xd = dev(x)
    yd = empty_bytes(3 * 36 * 4)
    acp.acp_stream_reduce_rows("add", yd, encode("f32", xd, shape, packed_strides(shape), stage), stage, 2, 256, 6,
                               stream())
    kind = expect_kind("row reduction linear grid")
    y = host(yd, np.float32, shape[:-1])
    assert np.array_equal(y, REF.reduce_rows(x)), "row sums"
    say(f"row sums: {kind}")


def tile_sqrt():
    x = W.sqrt_tiles_f32(tiles=4096, seed=14)        # 4096 tiles of 32x32: a persistent linear tile grid, 4 trips
    shape, box = x.shape, (1, 32, 32)
    xd = dev(x)
    yd = empty_bytes(x.nbytes)
    st = packed_strides(shape)
    acp.acp_tile_ewise("sqrt", encode("f32", yd, shape, st, box), [encode("f32", xd, shape, st, box)], 256,
                       stream())
    kind = expect_kind("tile linear grid")
    y = host(yd, np.float32, shape)
    ref = REF.ewise("sqrt", [x], np.float32)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32)), "sqrt"
    say(f"tile sqrt: {kind}")


if __name__ == "__main__":
    say("env: " + " ".join(f"{k}={v}" for k, v in sorted(os.environ.items()) if k.startswith("ACP_")))
    fma_stream()
    binary_stream()
    row_sums()
    tile_sqrt()
    torch.cuda.synchronize()
    say("all ok")
