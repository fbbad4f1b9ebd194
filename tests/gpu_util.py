"""Helpers shared by the GPU tests: device buffers from numpy arrays, ulp
distances, and a stream handle for the C ABI."""
import numpy as np
import torch

import async_copy_pipelining_amd as acp

DEV = "cuda:0"


def dev(a: np.ndarray) -> torch.Tensor:
    """Device copy of a numpy array (raw bytes preserved)."""
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.uint8).reshape(-1).copy())
    return t.to(DEV)


def empty_bytes(n: int, fill: int = 0xA5) -> torch.Tensor:
    return torch.full((max(1, n),), fill, dtype=torch.uint8, device=DEV)


def host(t: torch.Tensor, dtype, shape=None) -> np.ndarray:
    torch.cuda.synchronize()
    a = t.cpu().numpy().view(dtype)
    return a.reshape(shape) if shape is not None else a


def stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def ulp_diff(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """|a - b| in units of the last place, via ordered integer encodings."""
    if a.dtype == np.float32:
        ia, ib = a.view(np.int32).astype(np.int64), b.view(np.int32).astype(np.int64)
        lim = 0x80000000
    else:
        ia, ib = a.view(np.int16).astype(np.int64), b.view(np.int16).astype(np.int64)
        lim = 0x8000
    ia = np.where(ia < 0, -(ia + lim), ia)
    ib = np.where(ib < 0, -(ib + lim), ib)
    return np.abs(ia - ib)


def packed_strides(shape):
    st, out = 1, []
    for ext in reversed(shape):
        out.append(st)
        st *= ext
    return tuple(reversed(out))


def encode(dtype, t: torch.Tensor, shape, strides, box, swizzle=acp.ACP_SWIZZLE_NONE, offset_bytes=0):
    return acp.acp_encode_tiled(dtype, t.data_ptr() + offset_bytes, shape, strides, box, swizzle)
