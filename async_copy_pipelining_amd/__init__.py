"""Python binding of the acp C ABI (``include/acp.h``): argument marshalling only.

Every function has the name of the C entry point it wraps and forwards to it
through ctypes; all work happens in ``libacp.so`` (hand-written HIP kernels
for gfx950).  Pointer arguments accept an ``int`` device address or any
object with ``data_ptr()`` (a torch tensor); stream arguments accept an
``int`` handle or an object with ``cuda_stream`` (a torch stream).  A non-OK
status raises ``AcpError`` carrying the status and ``acp_last_error()``.

Importing this package fails when ``libacp.so`` has not been built: there is
no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libacp.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is missing: build it with `python async_copy_pipelining_amd/build.py` "
        "(the HIP library is the only implementation)")

try:
    # torch bundles its own HIP runtime under the same soname; loading torch
    # first makes libacp.so bind to that copy, so torch-allocated memory and
    # streams and acp's launches live in one runtime.
    import torch  # noqa: F401
except ImportError:  # pragma: no cover - acp itself does not need torch
    pass

_lib = ctypes.CDLL(LIB_PATH)

# acp_status
ACP_OK, ACP_ERR_INVALID, ACP_ERR_DECLINED, ACP_ERR_UNSUPPORTED, ACP_ERR_LDS, ACP_ERR_HIP = range(6)
STATUS_NAMES = {0: "OK", 1: "INVALID", 2: "DECLINED", 3: "UNSUPPORTED", 4: "LDS", 5: "HIP"}
# acp_dtype
ACP_U8, ACP_U16, ACP_U32, ACP_U64, ACP_F16, ACP_F32 = range(6)
DTYPES = {"u8": ACP_U8, "u16": ACP_U16, "u32": ACP_U32, "u64": ACP_U64, "f16": ACP_F16, "f32": ACP_F32}
# acp_swizzle / acp_oob
ACP_SWIZZLE_NONE, ACP_SWIZZLE_32B, ACP_SWIZZLE_64B, ACP_SWIZZLE_128B = 0, 1, 2, 3
ACP_OOB_ZERO = 0
# acp_op
ACP_OP_ZERO, ACP_OP_SQRT, ACP_OP_EXP, ACP_OP_ADD, ACP_OP_MUL, ACP_OP_FMA, ACP_OP_COPY = range(7)
OPS = {"zero": ACP_OP_ZERO, "sqrt": ACP_OP_SQRT, "exp": ACP_OP_EXP, "add": ACP_OP_ADD,
       "mul": ACP_OP_MUL, "fma": ACP_OP_FMA, "copy": ACP_OP_COPY}
ACP_MAX_RANK = 5


class AcpError(RuntimeError):
    def __init__(self, status: int, reason: str):
        super().__init__(f"acp {STATUS_NAMES.get(status, status)}: {reason}")
        self.status = status
        self.reason = reason


class acp_tile_desc(ctypes.Structure):
    _fields_ = [("opaque", ctypes.c_ubyte * 256)]


class acp_plan_info(ctypes.Structure):
    _fields_ = [
        ("rank", ctypes.c_int32), ("desc_elem_bytes", ctypes.c_int32),
        ("dims", ctypes.c_int64 * ACP_MAX_RANK), ("strides", ctypes.c_int64 * ACP_MAX_RANK),
        ("box", ctypes.c_int32 * ACP_MAX_RANK),
        ("issues", ctypes.c_int32), ("n_issue_axes", ctypes.c_int32), ("n_image_axes", ctypes.c_int32),
        ("swizzle", ctypes.c_int32), ("promoted", ctypes.c_int32),
        ("threads", ctypes.c_int32), ("vec", ctypes.c_int32), ("vec_bytes", ctypes.c_int32),
        ("outer", ctypes.c_int32), ("tile_bytes", ctypes.c_int64), ("n_tiles", ctypes.c_int64),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int
_DESC_P = ctypes.POINTER(acp_tile_desc)

_SIGS = {
    "acp_abi_version": ([], _I),
    "acp_last_error": ([], ctypes.c_char_p),
    "acp_last_kernel": ([], ctypes.c_char_p),
    "acp_encode_tiled": ([_DESC_P, _I, _I, _P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64),
                          ctypes.POINTER(ctypes.c_int32), _I, _I], _I),
    "acp_plan_query": ([_DESC_P, _I, _I, ctypes.POINTER(acp_plan_info)], _I),
    "acp_tile_copy": ([_DESC_P, _DESC_P, _I, _P], _I),
    "acp_tile_ewise": ([_I, _DESC_P, ctypes.POINTER(_DESC_P), _I, _I, _P], _I),
    "acp_stream_ewise": ([_I, _DESC_P, _DESC_P, _P, _P, ctypes.POINTER(ctypes.c_int32), _I, _I, _I, _P], _I),
    "acp_tile_reduce": ([_I, _DESC_P, _DESC_P, _I, _P], _I),
    "acp_stream_reduce_rows": ([_I, _P, _DESC_P, ctypes.POINTER(ctypes.c_int32), _I, _I, _I, _P], _I),
    "acp_stream_binary": ([_I, _DESC_P, _DESC_P, _DESC_P, ctypes.POINTER(ctypes.c_int32), _I, _I, _I, _I, _P], _I),
    "acp_debug_lds_image": ([_DESC_P, ctypes.c_int64, _I, _P, _P], _I),
    "acp_debug_ring_trace": ([_I, _I, _I, _I, _P, _P], _I),
    "acp_debug_stream_copy": ([_P, _P, ctypes.c_int64, _I, _P], _I),
    "acp_debug_stream_copy_shape": ([_P, _P, ctypes.c_int64, _I, _I, _I, _I, _I, _P], _I),
    "acp_debug_copy_tiles": ([_P, _P, _I, _P, _P, _P, _I, _I, _I, _P], _I),
    "acp_debug_stream_read": ([_P, ctypes.c_int64, _P, _I, _P], _I),
    "acp_debug_stream_fill": ([_P, ctypes.c_int64, ctypes.c_uint32, _I, _P], _I),
    "acp_debug_stream_widen": ([_P, _P, ctypes.c_int64, _I, _P], _I),
    "acp_debug_widen_tiles": ([_P, _P, _P, _P, _P, _P, _P], _I),
}
for _name, (_args, _res) in _SIGS.items():
    _fn = getattr(_lib, _name)
    _fn.argtypes = _args
    _fn.restype = _res

EXPORTED = tuple(_SIGS)


def _ptr(x) -> int | None:
    if x is None:
        return None
    if hasattr(x, "data_ptr"):
        return int(x.data_ptr())
    return int(x)


def _stream(s) -> int | None:
    if s is None:
        return None
    if hasattr(s, "cuda_stream"):
        return int(s.cuda_stream)
    return int(s)


def _check(status: int) -> None:
    if status != ACP_OK:
        raise AcpError(status, _lib.acp_last_error().decode())


def acp_last_kernel() -> str:
    return _lib.acp_last_kernel().decode()


def acp_abi_version() -> int:
    return int(_lib.acp_abi_version())


def acp_last_error() -> str:
    return _lib.acp_last_error().decode()


def acp_encode_tiled(dtype, gbase, shape, strides, box, swizzle=ACP_SWIZZLE_NONE, oob=ACP_OOB_ZERO) -> acp_tile_desc:
    dt = DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
    r = len(shape)
    d = acp_tile_desc()
    _check(_lib.acp_encode_tiled(ctypes.byref(d), dt, r, _ptr(gbase), (ctypes.c_int64 * r)(*shape),
                                 (ctypes.c_int64 * r)(*strides), (ctypes.c_int32 * r)(*box), int(swizzle), int(oob)))
    return d


def acp_plan_query(desc: acp_tile_desc, threads: int = 0, copy_only: bool = True) -> dict:
    info = acp_plan_info()
    _check(_lib.acp_plan_query(ctypes.byref(desc), int(threads), 1 if copy_only else 0, ctypes.byref(info)))
    r = info.rank
    return {
        "rank": r, "desc_elem_bytes": info.desc_elem_bytes,
        "dims": list(info.dims[:r]), "strides": list(info.strides[:r]), "box": list(info.box[:r]),
        "issues": info.issues, "n_issue_axes": info.n_issue_axes, "n_image_axes": info.n_image_axes,
        "swizzle": info.swizzle, "promoted": bool(info.promoted), "threads": info.threads,
        "vec": info.vec, "vec_bytes": info.vec_bytes, "outer": info.outer,
        "tile_bytes": info.tile_bytes, "n_tiles": info.n_tiles,
    }


def acp_tile_copy(src: acp_tile_desc, dst: acp_tile_desc, threads: int, stream=None) -> None:
    _check(_lib.acp_tile_copy(ctypes.byref(src), ctypes.byref(dst), int(threads), _stream(stream)))


def acp_tile_ewise(op, out: acp_tile_desc, ins, threads: int, stream=None) -> None:
    opc = OPS[op] if isinstance(op, str) else int(op)
    arr = (_DESC_P * max(1, len(ins)))(*[ctypes.pointer(d) for d in ins])
    _check(_lib.acp_tile_ewise(opc, ctypes.byref(out), arr, len(ins), int(threads), _stream(stream)))


def acp_stream_ewise(op, out: acp_tile_desc, x: acp_tile_desc, row_a, row_b, stage_box, stages: int,
                     threads: int, workgroups: int = 0, stream=None) -> None:
    opc = OPS[op] if isinstance(op, str) else int(op)
    sb = (ctypes.c_int32 * len(stage_box))(*stage_box)
    _check(_lib.acp_stream_ewise(opc, ctypes.byref(out), ctypes.byref(x), _ptr(row_a), _ptr(row_b), sb,
                                 int(stages), int(threads), int(workgroups), _stream(stream)))


def acp_tile_reduce(op, dst: acp_tile_desc, src: acp_tile_desc, threads: int, stream=None) -> None:
    opc = OPS[op] if isinstance(op, str) else int(op)
    _check(_lib.acp_tile_reduce(opc, ctypes.byref(dst), ctypes.byref(src), int(threads), _stream(stream)))


def acp_stream_reduce_rows(op, out, x: acp_tile_desc, stage_box, stages: int, threads: int, workgroups: int = 0,
                           stream=None) -> None:
    opc = OPS[op] if isinstance(op, str) else int(op)
    sb = (ctypes.c_int32 * len(stage_box))(*stage_box)
    _check(_lib.acp_stream_reduce_rows(opc, _ptr(out), ctypes.byref(x), sb, int(stages), int(threads),
                                       int(workgroups), _stream(stream)))


STAGING = {"ring": 0, "set": 1}


def acp_stream_binary(op, out: acp_tile_desc, x: acp_tile_desc, z: acp_tile_desc, stage_box, stages: int,
                      threads: int, workgroups: int = 0, z_staging="ring", stream=None) -> None:
    opc = OPS[op] if isinstance(op, str) else int(op)
    stg = STAGING[z_staging] if isinstance(z_staging, str) else int(z_staging)
    sb = (ctypes.c_int32 * len(stage_box))(*stage_box)
    _check(_lib.acp_stream_binary(opc, ctypes.byref(out), ctypes.byref(x), ctypes.byref(z), sb, int(stages),
                                  int(threads), int(workgroups), stg, _stream(stream)))


def acp_debug_lds_image(src: acp_tile_desc, tile_index: int, threads: int, out_bytes, stream=None) -> None:
    _check(_lib.acp_debug_lds_image(ctypes.byref(src), int(tile_index), int(threads), _ptr(out_bytes),
                                    _stream(stream)))


def acp_debug_ring_trace(n_iters: int, stages: int, loads: int, stores: int, out_events, stream=None) -> None:
    _check(_lib.acp_debug_ring_trace(int(n_iters), int(stages), int(loads), int(stores), _ptr(out_events),
                                     _stream(stream)))


def acp_debug_stream_copy(dst, src, nbytes: int, workgroups: int = 0, stream=None) -> None:
    _check(_lib.acp_debug_stream_copy(_ptr(dst), _ptr(src), int(nbytes), int(workgroups), _stream(stream)))


def acp_debug_stream_copy_shape(dst, src, nbytes: int, workgroups: int, threads: int, unroll: int,
                                load_nt: int = 1, store_nt: int = 1, stream=None) -> None:
    _check(_lib.acp_debug_stream_copy_shape(_ptr(dst), _ptr(src), int(nbytes), int(workgroups), int(threads),
                                            int(unroll), int(load_nt), int(store_nt), _stream(stream)))


def acp_debug_copy_tiles(dst, src, esize: int, shape, src_strides, box, tiles_per_trip: int = 2, threads: int = 128,
                         workgroups: int = 0, stream=None) -> None:
    arr64 = ctypes.c_int64 * 3
    arr32 = ctypes.c_int32 * 3
    _check(_lib.acp_debug_copy_tiles(_ptr(dst), _ptr(src), int(esize), arr64(*shape), arr64(*src_strides),
                                     arr32(*box), int(tiles_per_trip), int(threads), int(workgroups), _stream(stream)))


def acp_debug_stream_read(src, nbytes: int, sums, workgroups: int = 0, stream=None) -> None:
    _check(_lib.acp_debug_stream_read(_ptr(src), int(nbytes), _ptr(sums), int(workgroups), _stream(stream)))


def acp_debug_stream_fill(dst, nbytes: int, pattern: int, workgroups: int = 0, stream=None) -> None:
    _check(_lib.acp_debug_stream_fill(_ptr(dst), int(nbytes), int(pattern) & 0xFFFFFFFF, int(workgroups),
                                      _stream(stream)))


def acp_debug_stream_widen(dst, src, elements: int, workgroups: int = 0, stream=None) -> None:
    _check(_lib.acp_debug_stream_widen(_ptr(dst), _ptr(src), int(elements), int(workgroups), _stream(stream)))


def acp_debug_widen_tiles(dst, src, shape, src_strides, box, stage_box, stream=None) -> None:
    arr64, arr32 = ctypes.c_int64 * 5, ctypes.c_int32 * 5
    _check(_lib.acp_debug_widen_tiles(_ptr(dst), _ptr(src), arr64(*shape), arr64(*src_strides), arr32(*box),
                                      arr32(*stage_box), _stream(stream)))
