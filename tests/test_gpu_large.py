"""Tensors past 4 GiB: stage and tile bases beyond 2^32 bytes (64-bit
addressing, 32-bit buffer ranges clamped per stage).  The input is a
deterministic pattern written on the device (x[i] = (i mod 4093) / 4, exact
in float32); sampled rows are compared with the oracle, and the last row is
always among them."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import async_copy_pipelining_amd as acp  # noqa: E402
from oracle import reference as REF  # noqa: E402
from tests.gpu_util import encode, packed_strides, stream  # noqa: E402

ROWS, COLS = 1_310_720, 1024          # 5 GiB of float32


def say(msg):
    print(f"[gpu] {msg}", flush=True)


def _pattern_rows(rows: np.ndarray) -> np.ndarray:
    idx = rows[:, None].astype(np.int64) * COLS + np.arange(COLS, dtype=np.int64)[None, :]
    return ((idx % 4093).astype(np.float32) / np.float32(4.0)).astype(np.float32)


@pytest.fixture(scope="module")
def big_input():
    say(f"writing a {ROWS}x{COLS} float32 pattern on the device")
    n = ROWS * COLS
    x = torch.empty(n, dtype=torch.float32, device="cuda:0")
    chunk = 1 << 28
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        x[s:e] = (torch.arange(s, e, device="cuda:0", dtype=torch.int64) % 4093).to(torch.float32) / 4.0
    torch.cuda.synchronize()
    yield x
    del x
    torch.cuda.empty_cache()


def _sampled_rows(seed=0, k=300):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([rng.integers(0, ROWS, k), [0, ROWS - 1, (1 << 20) + 5]]))


@pytest.mark.parametrize("stage_box,box,workgroups,kind", [
    ((4, 1024), (4, 1024), 256, "stream linear grid"),   # persistent linear grid
    ((2, 512), (4, 1024), 0, "general stream"),          # one workgroup per 4x1024 tile, sub-stages
])
def test_stream_sqrt_past_4_gib(big_input, stage_box, box, workgroups, kind):
    say(f"stream sqrt over 5 GiB, stage {stage_box} box {box} workgroups {workgroups}")
    shape = (ROWS, COLS)
    y = torch.empty_like(big_input)
    st = packed_strides(shape)
    xdesc = encode("f32", big_input, shape, st, box)
    ydesc = encode("f32", y, shape, st, box)
    acp.acp_stream_ewise("sqrt", ydesc, xdesc, None, None, stage_box, 3, 256, workgroups, stream())
    assert acp.acp_last_kernel().startswith(kind)
    torch.cuda.synchronize()
    rows = _sampled_rows()
    got = y.view(ROWS, COLS)[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    want = REF.ewise("sqrt", [_pattern_rows(rows)], np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    del y


def test_tile_copy_past_4_gib(big_input):
    shape, box = (ROWS, COLS), (64, 64)          # 327 680 tiles of 16 KiB, a persistent grid
    say(f"tile copy over 5 GiB, box {box}")
    y = torch.empty_like(big_input)
    st = packed_strides(shape)
    acp.acp_tile_copy(encode("f32", big_input, shape, st, box), encode("f32", y, shape, st, box), 256, stream())
    torch.cuda.synchronize()
    rows = _sampled_rows(1)
    got = y.view(ROWS, COLS)[torch.from_numpy(rows).to("cuda:0")].cpu().numpy()
    assert np.array_equal(got.view(np.uint32), _pattern_rows(rows).view(np.uint32))
    del y
