#!/usr/bin/env python3
"""Throughput of the pipelined tile copy + elementwise path on one MI355X.

Default run: y = a[row] * x + b[row] over a [128, 500, 1024] float32 tensor
streamed through a 4-stage LDS ring (stage = two 1024-element rows, 256
threads, one persistent workgroup per CU), the configuration the HBM-roofline
target is quoted on.  One step = one launch of acp_stream_ewise over the whole
tensor.  The same line reports the 2-, 3- and 4-stage rings ("ring_stages"),
a plain register-path copy of the same bytes on the same device and the
ring's fraction of it ("copy_reference"),
the other workloads ("configs": the swizzled 8x256 tile copy, the 32x32 tile
sqrt, the 128x32 tile copy and the rank-5 exp stream, each with its roofline
figures, a plain copy of its bytes with its own walk ("reference") and its
own CPU-oracle baseline) and the CPU oracle of the streamed
fma.  Inputs are seeded synthetic tensors resident in HBM; three buffer sets
are rotated so that consecutive steps never hit data left in the 256 MB
last-level cache by the previous one.

Prints ONE JSON line with the metric, the roofline of the kernel (its average
launch duration from HIP events around the timed region, on the stream it
runs on) and the CPU oracle timed on a bounded sample of the same workload.

Other modes (measurement aids):
  --workload NAME   one workload alone (c1 c2 c3 c5, the references copy_ref /
                    read_ref / write_ref / widen_ref / widen_tiles_ref / tiles_copy_ref /
                    tile_ref, calib,
                    and pointwise / reduce / rowsum)
  --fixed-cost      the streamed fma and the reference copy over 1..128 slabs of
                    the tensor: per-launch fixed cost and per-byte rate of each
  --copy-sweep      plain register-path copies of the c4 bytes in 10 workgroup
                    shapes x 4 grids, and the reference shape under every pair
                    of load / store cache policies
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
METRIC = "achieved HBM GB/s (and % of peak) for pipelined tile copy+ewise, 1 MI355X"
PEAK_GBS = 8000.0
KERNEL_SOURCES = ["acp_dev_base.hpp", "acp_dev_ops.hpp", "acp_dev_map.hpp", "acp_dev_engine.hpp", "acp_dev_lin.hpp",
                  "acp_dev_gen.hpp", "acp_engine_impl.hpp", "acp_engine.hpp", "acp_k_stream_f32.hip",
                  "acp_k_stream_f16.hip", "acp_k_tile.hip", "acp_k_tile_gen.hip", "acp_k_tile_lin.hip",
                  "acp_k_copy.hip", "acp_k_ref.hip", "acp_engine.hip", "acp_api.cpp"]


def _code_only(text: str) -> str:
    """The source with comments removed and whitespace collapsed: a change
    to comments alone leaves the kernels, and so the hash, unchanged."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "async_copy_pipelining_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def _profile_field(workload_key: str, field: str):
    """A number from the committed rocprofv3 summary of a workload, or None
    when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{workload_key}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", txt)
    m_val = re.search(rf"{field}:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_val or m_hash.group(1) != kernel_hash():
        return None
    return float(m_val.group(1))


def traffic_from_profiles(workload_key: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, calibrated) from the
    committed summary of the workload."""
    return _profile_field(workload_key, "hbm_bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=None,
                    choices=["c1", "c2", "c3", "c4", "c5", "calib", "copy_ref", "read_ref", "write_ref", "widen_ref",
                             "widen_tiles_ref", "tiles_copy_ref", "tile_ref", "pointwise",
                             "reduce", "rowsum"],
                    help="measure one workload alone (default: c4 with ring_stages and configs); calib: torch's "
                         "copy of 256 MiB, the known-size kernel that scales HBM counters; copy_ref / read_ref / "
                         "write_ref: the library's register-path reference streams over the c4 tensor; "
                         "widen_ref: a contiguous f16 -> f32 widening stream; widen_tiles_ref / tiles_copy_ref / "
                         "tile_ref: plain copies with the walks of c5, c3 and c1")
    ap.add_argument("--stages", type=int, default=None,
                    help="ring slots (default: the measured best per workload; c4 and c5: 4)")
    ap.add_argument("--z-staging", default="ring", choices=["ring", "set"],
                    help="pointwise: how the second tensor reaches the ring")
    ap.add_argument("--reduce-over-batch", action="store_true",
                    help="reduce: add all 128 slabs into one [500,1024] destination (else slab by slab)")
    ap.add_argument("--rows", type=int, default=None,
                    help="rows per ring stage or tile (default per workload: c4 2, pointwise / reduce / rowsum 4, "
                         "reduce --reduce-over-batch 2)")
    ap.add_argument("--threads", type=int, default=None, help="threads per workgroup (default 256; c3 128; c1 64)")
    ap.add_argument("--workgroups", type=int, default=None,
                    help="persistent workgroups (default 256 x --wg-per-cu; 0: one workgroup per tile; c5 default 0)")
    ap.add_argument("--wg-per-cu", type=int, default=1)
    ap.add_argument("--c5-stage", default="1,1,1,64,64", help="c5: the stage box (outermost first)")
    ap.add_argument("--c5-box", default="1,2,16,64,64", help="c5: the tile box (outermost first)")
    ap.add_argument("--c5-swizzle", type=int, default=128, choices=[0, 32, 64, 128],
                    help="c5: the LDS swizzle span in bytes (0: none)")
    ap.add_argument("--sets", type=int, default=3, help="rotated buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=8.0, help="budget of the streamed-fma oracle sample")
    ap.add_argument("--config-cpu-seconds", type=float, default=2.0, help="budget of each config's oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ring-sweep", action="store_true", help="c4: skip the 2/3-stage report")
    ap.add_argument("--no-configs", action="store_true", help="default run: skip the other workloads")
    ap.add_argument("--fixed-cost", action="store_true",
                    help="fit launch time = fixed + bytes / rate over 1..128 slabs (streamed fma, reference copy)")
    ap.add_argument("--copy-sweep", action="store_true",
                    help="plain register-path copies of 262 MB in other shapes, cache policies and grids")
    args = ap.parse_args()
    return args


def _packed(shape):
    st, out = 1, []
    for e in reversed(shape):
        out.append(st)
        st *= e
    return tuple(reversed(out))


class Ctx:
    """Device plumbing shared by the workload builders."""

    def __init__(self, args):
        import numpy as np
        import torch

        import async_copy_pipelining_amd as acp
        import workloads as W
        self.np, self.torch, self.acp, self.W, self.args = np, torch, acp, W, args
        self.dev = "cuda:0"
        torch.cuda.set_device(0)
        self.stream = torch.cuda.current_stream()

    def to_dev(self, a):
        np = self.np
        return self.torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to(self.dev)

    def empty(self, nbytes):
        return self.torch.empty(int(nbytes), dtype=self.torch.uint8, device=self.dev)


def build(name, ctx, stages=None):
    """Launch callables (one per buffer set) and the accounting of one
    workload: algorithmic bytes per launch, the compute dtype, the config and
    the key of its committed profile summary."""
    args, acp, W, np, stream = ctx.args, ctx.acp, ctx.W, ctx.np, ctx.stream
    sets = args.sets
    launches, unit = [], "GB/s"
    wpc = args.wg_per_cu
    G = 256 * wpc if args.workgroups is None else args.workgroups
    if name == "c4":
        rows = args.rows or 2
        S = stages or args.stages or 4
        threads = args.threads or 256
        shape, stage = (128, 500, 1024), (1, rows, 1024)
        x, a, b = W.fma_rows_f32(shape, seed=4)
        for _ in range(sets):
            xd, ad, bd, yd = ctx.to_dev(x), ctx.to_dev(a), ctx.to_dev(b), ctx.empty(x.nbytes)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, _packed(shape), stage)
            ydesc = acp.acp_encode_tiled("f32", yd, shape, _packed(shape), stage)
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, ad=ad, bd=bd, keep=(xd, yd):
                            acp.acp_stream_ewise("fma", ydesc, xdesc, ad, bd, stage, launches_stages[0], threads, G,
                                                 stream))
        launches_stages = [S]
        out = dict(bytes=x.nbytes * 2 + a.nbytes + b.nbytes, dtype="f32",
                   config={"workload": f"stream fma y=a[row]*x+b[row], [128,500,1024] f32, {S}-stage LDS ring, "
                                       f"stage (1,{rows},1024)", "shape": list(shape), "stages": S,
                           "stage_box": list(stage), "threads": threads, "workgroups": G},
                   key=f"stream_fma_f32_128x500x1024_s{S}_r{rows}")
        out["set_stages"] = launches_stages      # the ring sweep changes the slot count in place
    elif name == "c1":
        # one 8x256 f16 tile through the 128-byte swizzled LDS image and back,
        # 64 threads: latency-bound, so the figure that matters is the launch
        # time in microseconds
        threads = args.threads or 64
        x = W.tile_bits_f16((8, 256), seed=1)
        shape = x.shape
        for _ in range(sets):
            xd, yd = ctx.to_dev(x), ctx.empty(x.nbytes)
            xdesc = acp.acp_encode_tiled("f16", xd, shape, _packed(shape), shape, acp.ACP_SWIZZLE_128B)
            ydesc = acp.acp_encode_tiled("f16", yd, shape, _packed(shape), shape, acp.ACP_SWIZZLE_128B)
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_tile_copy(xdesc, ydesc, threads, stream))
        unit = "us"
        out = dict(bytes=x.nbytes * 2, dtype="f16",
                   config={"workload": f"swizzled tile copy, one 8x256 f16 tile (128-byte swizzle), {threads} "
                                       "threads (latency-bound: microseconds per launch)"},
                   key="tile_copy_swizzled_f16_8x256")
    elif name == "tile_ref":
        # the latency floor beside c1: a plain register-path copy of the same
        # 4 KiB by one 64-thread workgroup (16-byte loads, then stores), no LDS
        x = W.tile_bits_f16((8, 256), seed=1)
        for _ in range(sets):
            xd, yd = ctx.to_dev(x), ctx.empty(x.nbytes)
            launches.append(lambda xd=xd, yd=yd:
                            acp.acp_debug_stream_copy_shape(yd, xd, x.nbytes, 1, 64, 16, 1, 1, stream))
        unit = "us"
        out = dict(bytes=x.nbytes * 2, dtype="f16",
                   config={"workload": "reference register-path copy of one 8x256 f16 tile (4 KiB), one workgroup "
                                       "of 64 threads, no LDS (latency-bound: microseconds per launch)"},
                   key="tile_copy_reference_4KiB")
    elif name == "c2":
        threads = args.threads or 256
        x = W.sqrt_tiles_f32(65536, seed=2)
        shape = x.shape
        for _ in range(sets):
            xd, yd = ctx.to_dev(x), ctx.empty(x.nbytes)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, _packed(shape), (1, 32, 32))
            ydesc = acp.acp_encode_tiled("f32", yd, shape, _packed(shape), (1, 32, 32))
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_tile_ewise("sqrt", ydesc, [xdesc], threads, stream))
        out = dict(bytes=x.nbytes * 2, dtype="f32",
                   config={"workload": f"tile sqrt, 65536 tiles of 32x32 f32, {threads} threads, persistent grid"},
                   key="tile_sqrt_f32_65536x32x32")
    elif name == "c3":
        threads = args.threads or 128
        shape = (128, 500, 1024)
        x = W.normal_f16(shape, seed=3)
        for _ in range(sets):
            xd, yd = ctx.to_dev(x), ctx.empty(x.nbytes)
            xdesc = acp.acp_encode_tiled("f16", xd, shape, _packed(shape), (1, 128, 32))
            ydesc = acp.acp_encode_tiled("f16", yd, shape, _packed(shape), (1, 128, 32))
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_tile_copy(xdesc, ydesc, threads, stream))
        out = dict(bytes=x.nbytes * 2, dtype="f16",
                   config={"workload": f"tile copy, [128,500,1024] f16, 128x32 tiles, {threads} threads"},
                   key="tile_copy_f16_128x500x1024")
    elif name == "tiles_copy_ref":
        threads = args.threads or 128
        shape = (128, 500, 1024)
        x = W.normal_f16(shape, seed=3)
        for _ in range(sets):
            xd, yd = ctx.to_dev(x), ctx.empty(x.nbytes)
            launches.append(lambda xd=xd, yd=yd: acp.acp_debug_copy_tiles(
                yd, xd, 2, shape, _packed(shape), (1, 128, 32), 2, threads, G, stream))
        out = dict(bytes=x.nbytes * 2, dtype="f16",
                   config={"workload": f"reference register-path copy with the tile copy's walk: [128,500,1024] "
                                       f"f16, 128x32 tiles in pairs along the rows, blocked runs of consecutive "
                                       f"pairs per workgroup, {threads} threads, {G} workgroups, two pairs in "
                                       f"flight, no LDS, no ring"},
                   key="tile_copy_reference_f16_128x500x1024")
    elif name == "c5":
        threads = args.threads or 256
        S = stages or args.stages or 4
        shape, pitch = (4, 8, 64, 128, 256), 264
        c5_stage = tuple(int(v) for v in args.c5_stage.split(","))
        c5_box = tuple(int(v) for v in args.c5_box.split(","))
        c5_swz = {0: acp.ACP_SWIZZLE_NONE, 32: acp.ACP_SWIZZLE_32B, 64: acp.ACP_SWIZZLE_64B,
                  128: acp.ACP_SWIZZLE_128B}[args.c5_swizzle]
        c5_wgs = 0 if args.workgroups is None else args.workgroups
        storage, strides = W.padded_uniform_f16(shape, pitch=pitch, seed=5)
        n = int(np.prod(shape))
        for _ in range(sets):
            xd, yd = ctx.to_dev(storage), ctx.empty(n * 4)
            xdesc = acp.acp_encode_tiled("f16", xd, shape, strides, c5_box, c5_swz)
            ydesc = acp.acp_encode_tiled("f32", yd, shape, _packed(shape), c5_box)
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_stream_ewise("exp", ydesc, xdesc, None, None, c5_stage, S, threads, c5_wgs,
                                                 stream))
        out = dict(bytes=n * 2 + n * 4, dtype="f16->f32",
                   config={"workload": f"rank-5 exp (4,8,64,128,256) f16 pitch 264 -> f32, box {c5_box}, "
                                       f"{S}-stage ring, {args.c5_swizzle}-byte swizzle, stage {c5_stage}"},
                   key=f"stream_exp_rank5_s{S}" + ("" if args.c5_swizzle == 128 else f"_swz{args.c5_swizzle}"))
    elif name == "pointwise":
        rows, S, threads = args.rows or 4, args.stages or 2, args.threads or 256
        shape, stage = (128, 500, 1024), (1, rows, 1024)
        rng = np.random.default_rng(6)
        x = rng.standard_normal(shape, dtype=np.float32)
        z = rng.standard_normal(shape, dtype=np.float32)
        for _ in range(sets):
            xd, zd, yd = ctx.to_dev(x), ctx.to_dev(z), ctx.empty(x.nbytes)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, _packed(shape), stage)
            zdesc = acp.acp_encode_tiled("f32", zd, shape, _packed(shape), stage)
            ydesc = acp.acp_encode_tiled("f32", yd, shape, _packed(shape), stage)
            launches.append(lambda xdesc=xdesc, zdesc=zdesc, ydesc=ydesc, keep=(xd, zd, yd):
                            acp.acp_stream_binary("add", ydesc, xdesc, zdesc, stage, S, threads, G, args.z_staging,
                                                  stream))
        out = dict(bytes=3 * x.nbytes, dtype="f32",
                   config={"workload": f"two-tensor stream y = x + z, [128,500,1024] f32, {S}-stage LDS ring, "
                                       f"stage (1,{rows},1024), z staged '{args.z_staging}'", "workgroups": G},
                   key=f"stream_add2_f32_128x500x1024_s{S}_r{rows}_{args.z_staging}")
    elif name == "reduce":
        # store with reduce-add of a [128,500,1024] f32 tensor in (1,R,1024)
        # tiles: into a same-shape destination (one contribution per element)
        # or into one [1,500,1024] slab (128 contributions per element)
        threads = args.threads or 256
        rows = args.rows or (2 if args.reduce_over_batch else 4)
        shape = (128, 500, 1024)
        dshape = (1, 500, 1024) if args.reduce_over_batch else shape
        box = (1, rows, 1024)
        rng = np.random.default_rng(7)
        x = rng.standard_normal(shape, dtype=np.float32)
        for _ in range(sets):
            xd = ctx.to_dev(x)
            yd = ctx.torch.zeros(int(np.prod(dshape)) * 4, dtype=ctx.torch.uint8, device=ctx.dev)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, _packed(shape), box)
            ydesc = acp.acp_encode_tiled("f32", yd, dshape, _packed(dshape), box)
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_tile_reduce("add", ydesc, xdesc, threads, stream))
        # algorithmic bytes: the source once, the destination read and written once
        out = dict(bytes=x.nbytes + 2 * int(np.prod(dshape)) * 4, dtype="f32",
                   config={"workload": f"store with reduce-add, [128,500,1024] f32 tiles (1,{rows},1024) into "
                                       f"{list(dshape)}"},
                   key=f"tile_reduce_f32_128x500x1024_r{rows}_{'batch' if args.reduce_over_batch else 'slab'}")
    elif name == "rowsum":
        rows, S, threads = args.rows or 4, args.stages or 2, args.threads or 256
        shape, stage = (128, 500, 1024), (1, rows, 1024)
        rng = np.random.default_rng(8)
        x = rng.standard_normal(shape, dtype=np.float32)
        for _ in range(sets):
            xd, yd = ctx.to_dev(x), ctx.empty(128 * 500 * 4)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, _packed(shape), stage)
            launches.append(lambda xdesc=xdesc, keep=(xd, yd):
                            acp.acp_stream_reduce_rows("add", keep[1], xdesc, stage, S, threads, G, stream))
        out = dict(bytes=x.nbytes + 128 * 500 * 4, dtype="f32",
                   config={"workload": f"row sums of [128,500,1024] f32 -> [128,500], {S}-stage LDS ring, "
                                       f"stage (1,{rows},1024)", "workgroups": G},
                   key=f"stream_rowsum_f32_128x500x1024_s{S}_r{rows}")
    elif name == "widen_ref":
        n = 4 * 8 * 64 * 128 * 256            # the rank-5 exp workload's element count, packed
        for _ in range(sets):
            xd = ctx.torch.zeros(n * 2, dtype=ctx.torch.uint8, device=ctx.dev)
            yd = ctx.empty(n * 4)
            launches.append(lambda xd=xd, yd=yd: acp.acp_debug_stream_widen(yd, xd, n, G, stream))
        out = dict(bytes=n * 6, dtype="f16->f32",
                   config={"workload": f"reference register-path f16 -> f32 widening stream of {n} elements "
                                       f"(the rank-5 exp workload's count, packed), {G} workgroups"},
                   key="stream_widen_reference_67M")
    elif name == "widen_tiles_ref":
        # the rank-5 exp workload's walk (tiles (1,2,16,64,64), stages
        # (1,1,1,64,64), row pitch 264) as a plain register-path widening copy
        shape, pitch = (4, 8, 64, 128, 256), 264
        storage, strides = W.padded_uniform_f16(shape, pitch=pitch, seed=5)
        n = int(np.prod(shape))
        for _ in range(sets):
            xd, yd = ctx.to_dev(storage), ctx.empty(n * 4)
            launches.append(lambda xd=xd, yd=yd: acp.acp_debug_widen_tiles(
                yd, xd, shape, strides, (1, 2, 16, 64, 64), (1, 1, 1, 64, 64), stream))
        out = dict(bytes=n * 6, dtype="f16->f32",
                   config={"workload": "reference register-path widening copy with the rank-5 exp workload's walk: "
                                       "(4,8,64,128,256) f16 pitch 264 -> f32, tiles (1,2,16,64,64), stages "
                                       "(1,1,1,64,64), one workgroup per tile"},
                   key="widen_tiles_reference_rank5")
    elif name in ("copy_ref", "read_ref", "write_ref"):
        nbytes = 128 * 500 * 1024 * 4
        # Reads alone need more bytes in flight than one 16 KiB batch per CU:
        # the read-only stream runs two workgroups per CU by default.
        Gr = 2 * G if args.workgroups is None else G
        for _ in range(sets):
            xd = ctx.torch.ones(nbytes, dtype=ctx.torch.uint8, device=ctx.dev)
            yd = ctx.empty(nbytes)
            sums = ctx.empty(16 * 4096)
            if name == "copy_ref":
                launches.append(lambda xd=xd, yd=yd: acp.acp_debug_stream_copy(yd, xd, nbytes, G, stream))
            elif name == "read_ref":
                launches.append(lambda xd=xd, s=sums: acp.acp_debug_stream_read(xd, nbytes, s, Gr, stream))
            else:
                launches.append(lambda yd=yd: acp.acp_debug_stream_fill(yd, nbytes, 0x3F800000, G, stream))
        what = {"copy_ref": ("copy", 2 * nbytes, "stream_copy_reference_262MB"),
                "read_ref": ("read-only stream", nbytes, "stream_read_reference_262MB"),
                "write_ref": ("write-only stream", nbytes, "stream_write_reference_262MB")}[name]
        out = dict(bytes=what[1], dtype="u8",
                   config={"workload": f"reference register-path {what[0]} of 262144000 B (the c4 tensor), "
                                       f"{Gr if name == 'read_ref' else G} workgroups"},
                   key=what[2])
    elif name == "calib":
        nbytes = 256 << 20
        for _ in range(sets):
            xd = ctx.torch.ones(nbytes, dtype=ctx.torch.uint8, device=ctx.dev)
            yd = ctx.empty(nbytes)
            launches.append(lambda xd=xd, yd=yd: yd.copy_(xd))
        out = dict(bytes=2 * nbytes, dtype="u8",
                   config={"workload": "torch copy_ of 256 MiB (counter calibration: 268435456 B read, "
                                       "268435456 B written)"},
                   key="calib_copy_256MiB")
    else:
        raise ValueError(name)
    out["launches"] = launches
    out["unit"] = unit
    return out


def time_launches(ctx, fns, steps, warmup):
    """Average launch time (ms) of `steps` back-to-back launches after
    `warmup` untimed ones, from one event pair on the launch stream."""
    torch = ctx.torch
    for i in range(warmup):
        fns[i % len(fns)]()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(ctx.stream)
    for i in range(steps):
        fns[i % len(fns)]()
    t1.record(ctx.stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / steps


def bracketed_median(ctx, fns, steps):
    """Median of per-launch times, each launch between its own event pair
    (the dispatch gap is added to every launch)."""
    torch = ctx.torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    for i in range(steps):
        starts[i].record(ctx.stream)
        fns[i % len(fns)]()
        ends[i].record(ctx.stream)
    torch.cuda.synchronize()
    v = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
    return v[len(v) // 2]


def roofline(wl, avg_ms, median_ms):
    achieved = wl["bytes"] / (avg_ms * 1e-3) / 1e9
    return {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic_from_profiles(wl["key"]),
            "algorithmic_bytes_per_launch": wl["bytes"], "avg_launch_ms": round(avg_ms, 5),
            "median_event_bracketed_launch_ms": round(median_ms, 5), "kernel_source_hash": kernel_hash()}


def c1_graph_replay_us(ctx, steps):
    """The swizzled 8x256 tile copy with the host out of the loop: `steps`
    launches (rotating buffer sets) captured in one HIP graph on a side
    stream and replayed; microseconds per launch, and whether the replayed
    copies are bit-identical."""
    torch, acp, W = ctx.torch, ctx.acp, ctx.W
    x = W.tile_bits_f16((8, 256), seed=1)
    shape = x.shape
    bufs = [(ctx.to_dev(x), ctx.empty(x.nbytes)) for _ in range(ctx.args.sets)]
    descs = [(acp.acp_encode_tiled("f16", xd, shape, _packed(shape), shape, acp.ACP_SWIZZLE_128B),
              acp.acp_encode_tiled("f16", yd, shape, _packed(shape), shape, acp.ACP_SWIZZLE_128B)) for xd, yd in bufs]
    for xdesc, ydesc in descs:          # plan and cache the launches outside the capture
        acp.acp_tile_copy(xdesc, ydesc, 64, ctx.stream)
    torch.cuda.synchronize()
    for _, yd in bufs:
        yd.zero_()
    side = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(steps):
            xdesc, ydesc = descs[i % len(descs)]
            acp.acp_tile_copy(xdesc, ydesc, 64, h)
    g.replay()
    torch.cuda.synchronize()
    exact = all(torch.equal(xd, yd) for xd, yd in bufs)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    g.replay()
    t1.record()
    torch.cuda.synchronize()
    us = t0.elapsed_time(t1) * 1e3 / steps
    del g
    return round(us, 2), exact


def measure_config(name, ctx, steps, warmup):
    """One of the other workloads: its throughput (microseconds per launch for
    the latency-bound single tile), the launch the library chose, and its
    roofline figures."""
    wl = build(name, ctx)
    avg = time_launches(ctx, wl["launches"], steps, warmup)
    kernel = ctx.acp.acp_last_kernel()
    med = bracketed_median(ctx, wl["launches"], steps)
    rf = roofline(wl, avg, med)
    if wl["unit"] == "us":
        entry = {"value": round(avg * 1e3, 2), "unit": "us per launch", "back_to_back_us": round(avg * 1e3, 2),
                 "event_bracketed_median_us": round(med * 1e3, 2),
                 "kernel_us": _profile_field(wl["key"], "kernel_average_ns")}
        if name == "c1":
            entry["graph_replay_us"], entry["graph_replay_bit_exact"] = c1_graph_replay_us(ctx, steps)
        if entry["kernel_us"] is not None:
            entry["kernel_us"] = round(entry["kernel_us"] / 1e3, 2)
    else:
        entry = {"value": rf["achieved"], "unit": "GB/s", "frac": rf["frac"], "roofline": rf}
    entry.update({"ms_per_step": round(avg, 5), "dtype": wl["dtype"], "config": {**wl["config"], "kernel": kernel}})
    del wl
    ctx.torch.cuda.synchronize()
    ctx.torch.cuda.empty_cache()
    return entry


def progress(msg: str) -> None:
    """One line per measurement phase on stderr (stdout carries only the
    JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the path runs on one GPU only (each GPU would take its own slab; no "
                                   "collective is part of it): run with --gpus 1", "n_gpus": args.gpus}))
        sys.exit(2)
    ctx = Ctx(args)
    if args.fixed_cost:
        fixed_cost(ctx)
        return
    if args.copy_sweep:
        copy_sweep(ctx)
        return
    name = args.workload or "c4"
    progress(f"workload {name}: building inputs")
    wl = build(name, ctx)
    fns = wl["launches"]
    ring = None
    if name == "c4" and not args.no_ring_sweep:
        progress("ring sweep: 2, 3 and 4 slots")
        # the 2-, 3- and 4-stage rings, back to back like `value` (measured
        # before the headline's own warm-up and timed region)
        ring = {}
        for st in (2, 3, 4):
            wl["set_stages"][0] = st
            ring[str(st)] = round(wl["bytes"] / (time_launches(ctx, fns, args.steps, args.warmup) * 1e-3) / 1e9, 1)
        wl["set_stages"][0] = args.stages or 4

    # Timed region: warm-up, then K steps back to back, bracketed by
    # synchronize and one event pair on the launch stream.  One step is one
    # launch of the kernel, so the event pair's time over K is the kernel's
    # average launch duration (the figure rocprofv3's kernel trace reports per
    # dispatch, plus the dispatch gap).
    progress(f"timed region: {args.warmup} warm-up, {args.steps} steps")
    ms_per_step = time_launches(ctx, fns, args.steps, args.warmup)
    kernel = ctx.acp.acp_last_kernel()
    median = bracketed_median(ctx, fns, args.steps)
    rf = roofline(wl, ms_per_step, median)
    if wl["unit"] == "us":
        value, unit = round(ms_per_step * 1e3, 3), "us"
    else:
        value, unit = round(wl["bytes"] / (ms_per_step * 1e-3) / 1e9, 1), "GB/s"
    result = {
        "metric": METRIC if unit == "GB/s" else "microseconds per launch, swizzled 8x256 f16 tile copy, 1 MI355X",
        "value": value, "unit": unit, "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": unit == "GB/s", "scaling": "weak", "vs_baseline": None, "dtype": wl["dtype"],
        "data": "synthetic (seeded numpy draws resident in HBM, 3 rotated buffer sets)",
        "config": {**wl["config"], "kernel": kernel},
        "percent_of_peak": round(100.0 * rf["achieved"] / PEAK_GBS, 2),
        "roofline": rf,
    }
    if ring is not None:
        result["ring_stages"] = {"unit": "GB/s", **ring}
    del wl, fns
    ctx.torch.cuda.empty_cache()
    if name == "c4" and args.workload is None and not args.no_configs:
        # the same box's ceiling beside the headline: a plain register-path
        # copy (no LDS, no ring) of the same 262 MB read and written, timed
        # the same way
        progress("copy reference")
        ref = measure_config("copy_ref", ctx, args.steps, args.warmup)
        result["copy_reference"] = {"value": ref["value"], "unit": "GB/s", "frac": ref["frac"],
                                    "workload": ref["config"]["workload"],
                                    "ring_fraction_of_copy": round(value / ref["value"], 4)}
        configs = {}
        # each config beside a plain register-path copy of its bytes with its
        # walk (no LDS, no ring): the 4 KiB tile, the contiguous tensor, the
        # paired 128x32 tiles, the rank-5 tiles and stages
        walk_ref = {"c1": "tile_ref", "c2": "copy_ref", "c3": "tiles_copy_ref", "c5": "widen_tiles_ref"}
        for c in ("c1", "c2", "c3", "c5"):
            progress(f"config {c} and its reference")
            configs[c] = measure_config(c, ctx, args.steps, args.warmup)
            r = measure_config(walk_ref[c], ctx, args.steps, args.warmup)
            v, rv = configs[c]["value"], r["value"]
            configs[c]["reference"] = {"workload": r["config"]["workload"], "value": rv, "unit": r["unit"],
                                       "fraction": round(rv / v if r["unit"].startswith("us") else v / rv, 4)}
            if r.get("kernel_us") is not None:
                configs[c]["reference"]["kernel_us"] = r["kernel_us"]
            if not args.no_cpu_baseline:
                progress(f"config {c}: CPU oracle sample")
                configs[c]["cpu_baseline"] = cpu_baseline_config(c, args.config_cpu_seconds)
        result["configs"] = configs
    if not args.no_cpu_baseline:
        progress("CPU oracle samples")
        if name == "c4":
            result["cpu_baseline"] = cpu_baseline_c4(args.cpu_seconds)
            result["cpu_baseline_all_cores"] = cpu_baseline_c4_parallel(args.cpu_seconds)
        elif name in ("c1", "c2", "c3", "c5"):
            result["cpu_baseline"] = cpu_baseline_config(name, args.config_cpu_seconds)
    print(json.dumps(result), flush=True)


# ---------------------------------------------------------------------------
# Fixed cost per launch: the streamed fma (the default launch) and the
# reference copy over 1..128 [500,1024] slabs of the same tensors.  Windows of
# N slabs rotate through all three buffer sets so that no window is reused
# before more than the 256 MB last-level cache has been streamed; each launch
# is timed between its own event pair (device time: host gaps between
# launches are not counted).  A least-squares line time = fixed + bytes /
# rate over the slab counts gives each kernel's fixed cost and per-byte rate.

def _fit(points):
    n = len(points)
    mx = sum(p[0] for p in points) / n
    my = sum(p[1] for p in points) / n
    sxx = sum((p[0] - mx) ** 2 for p in points)
    sxy = sum((p[0] - mx) * (p[1] - my) for p in points)
    slope = sxy / sxx
    return my - slope * mx, slope


def fixed_cost(ctx):
    args, acp, W, np, torch = ctx.args, ctx.acp, ctx.W, ctx.np, ctx.torch
    shape = (128, 500, 1024)
    slab_b = 500 * 1024 * 4
    x, a, b = W.fma_rows_f32(shape, seed=4)
    bufs = [(ctx.to_dev(x), ctx.to_dev(a), ctx.to_dev(b), ctx.empty(x.nbytes)) for _ in range(3)]
    stage = (1, 2, 1024)
    res = {"workload": "streamed fma (stage (1,2,1024), 4 slots, 256 workgroups) and reference copy, "
                       "1..128 slabs of [500,1024] f32", "points": {}}
    for kind in ("ring", "copy"):
        pts = []
        for N in (1, 2, 4, 8, 16, 32, 64, 128):
            n_win = max(12, 3 * (128 // N))
            fns = []
            for j in range(n_win):
                xd, ad, bd, yd = bufs[j % 3]
                s0 = ((j // 3) * N) % (128 - N + 1)
                if kind == "ring":
                    sh = (N, 500, 1024)
                    xdesc = acp.acp_encode_tiled("f32", xd.data_ptr() + s0 * slab_b, sh, _packed(sh), stage)
                    ydesc = acp.acp_encode_tiled("f32", yd.data_ptr() + s0 * slab_b, sh, _packed(sh), stage)
                    pa, pb = ad.data_ptr() + s0 * 2000, bd.data_ptr() + s0 * 2000
                    fns.append(lambda xdesc=xdesc, ydesc=ydesc, pa=pa, pb=pb:
                               acp.acp_stream_ewise("fma", ydesc, xdesc, pa, pb, stage, 4, 256, 256, ctx.stream))
                else:
                    px, py = xd.data_ptr() + s0 * slab_b, yd.data_ptr() + s0 * slab_b
                    fns.append(lambda px=px, py=py, nb=N * slab_b:
                               acp.acp_debug_stream_copy(py, px, nb, 256, ctx.stream))
            warm = 2 * len(fns)
            for i in range(warm):
                fns[i % len(fns)]()
            torch.cuda.synchronize()
            steps = max(60, len(fns))
            starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
            for i in range(steps):
                starts[i].record(ctx.stream)
                fns[i % len(fns)]()
                ends[i].record(ctx.stream)
            torch.cuda.synchronize()
            t = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))
            med_us = t[len(t) // 2] * 1e3
            nbytes = N * (2 * slab_b + (1000 * 4 if kind == "ring" else 0))
            pts.append((nbytes, med_us))
            res["points"].setdefault(kind, []).append({"slabs": N, "bytes": nbytes, "median_us": round(med_us, 2),
                                                       "warmup_launches": warm, "timed_launches": steps})
        fixed, per_byte = _fit(pts)
        res[kind] = {"fixed_us": round(fixed, 2), "rate_GBps": round(1e-3 / per_byte, 1)}
    print(json.dumps(res), flush=True)


# ---------------------------------------------------------------------------
# Copy sweep: what a plain register-path copy of the reference copy's bytes
# reaches in other shapes (threads x 16-byte loads per lane), cache policies
# and grids, over the same rotated buffer sets as every workload.  The
# reference copy's own shape is 256 x 4 with non-temporal loads and stores.

COPY_SWEEP_SHAPES = ((256, 4), (256, 2), (256, 8), (512, 2), (512, 4), (512, 8), (1024, 2), (1024, 4),
                     (128, 8), (64, 16))
COPY_SWEEP_GRIDS = (256, 512, 1024, 4096)


def copy_sweep(ctx):
    args, acp, torch = ctx.args, ctx.acp, ctx.torch
    n = 262144000
    bufs = [(torch.full((n,), 1 + i, dtype=torch.uint8, device=ctx.dev), ctx.empty(n)) for i in range(args.sets)]
    points = []
    for threads, unroll in COPY_SWEEP_SHAPES:
        policies = ((1, 1), (1, 0), (0, 1), (0, 0)) if (threads, unroll) == (256, 4) else ((1, 1),)
        for lnt, snt in policies:
            for G in COPY_SWEEP_GRIDS:
                fns = [lambda x=x, y=y, G=G, t=threads, u=unroll, l=lnt, s=snt:
                       acp.acp_debug_stream_copy_shape(y, x, n, G, t, u, l, s, ctx.stream) for x, y in bufs]
                avg = time_launches(ctx, fns, args.steps, args.warmup)
                points.append({"threads": threads, "unroll": unroll, "load_nt": lnt, "store_nt": snt,
                               "workgroups": G, "avg_launch_us": round(avg * 1e3, 2),
                               "GBps": round(2 * n / (avg * 1e-3) / 1e9, 1)})
    print(json.dumps({"workload": "plain register-path copy of 262 144 000 B, shapes x cache policies x grids",
                      "sets": args.sets, "steps": args.steps, "warmup": args.warmup, "points": points}), flush=True)


# ---------------------------------------------------------------------------
# CPU baselines: the oracle's plain definition of each workload (as it
# stands, not tuned), timed on the host on a bounded sample of the same
# workload.

def cpu_baseline_c4(budget_s: float):
    """The oracle's streamed fma over whole [500, 1024] slabs of the same
    workload, slab after slab (wrapping around) until the time budget is
    spent; single-threaded numpy."""
    import numpy as np

    import workloads as W
    from oracle import reference as REF

    x, a, b = W.fma_rows_f32((128, 500, 1024), seed=4)
    done, t0 = 0, time.perf_counter()
    while True:
        k = done % 128
        REF.stream_ewise("fma", x[k], a[k], b[k], np.float32)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    nbytes = done * (500 * 1024 * 4 * 2 + 500 * 8)
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{done} [500,1024] f32 slabs of the streamed-fma workload ({done / 128:.2f} passes "
                      f"over the 128 slabs) in {el:.1f} s, numpy single thread"}


def cpu_baseline_config(name: str, budget_s: float):
    """The oracle's plain definition on a bounded sample of workload `name`
    (single thread): tile copy = the identity, tile sqrt and the rank-5 exp =
    the op element by element."""
    import numpy as np

    import workloads as W
    from oracle import reference as REF

    done, t0 = 0, time.perf_counter()
    if name == "c1":
        x = W.tile_bits_f16((8, 256), seed=1)
        while time.perf_counter() - t0 < budget_s:
            REF.tile_copy(x)
            done += 1
        el = time.perf_counter() - t0
        return {"value": round(el / done * 1e6, 3), "unit": "us per tile", "cores": 1, "kind": "oracle",
                "sample": f"{done} copies of the 8x256 f16 tile in {el:.1f} s (reference.tile_copy), numpy "
                          "single thread"}
    if name == "c2":
        x = W.sqrt_tiles_f32(65536, seed=2)
        chunk = 2048
        while time.perf_counter() - t0 < budget_s:
            k = (done * chunk) % 65536
            REF.ewise("sqrt", [x[k:k + chunk]], np.float32)
            done += 1
        el = time.perf_counter() - t0
        nbytes = done * chunk * 1024 * 8
        return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{done} chunks of {chunk} 32x32 f32 tiles of the tile-sqrt workload in {el:.1f} s "
                          "(reference.ewise sqrt), numpy single thread"}
    if name == "c3":
        x = W.normal_f16((128, 500, 1024), seed=3)
        while time.perf_counter() - t0 < budget_s:
            REF.tile_copy(x[done % 128])
            done += 1
        el = time.perf_counter() - t0
        nbytes = done * 500 * 1024 * 2 * 2
        return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{done} [500,1024] f16 slabs of the tile-copy workload in {el:.1f} s "
                          "(reference.tile_copy), numpy single thread"}
    if name == "c5":
        shape = (4, 8, 64, 128, 256)
        storage, strides = W.padded_uniform_f16(shape, pitch=264, seed=5)
        xv = W.strided_view(storage, shape, strides)
        while time.perf_counter() - t0 < budget_s:
            i = done % 32
            REF.stream_ewise("exp", xv[i // 8, i % 8], out_dtype=np.float32)
            done += 1
        el = time.perf_counter() - t0
        nbytes = done * 64 * 128 * 256 * 6
        return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
                "sample": f"{done} (64,128,256) blocks of the rank-5 exp workload in {el:.1f} s "
                          "(reference.stream_ewise exp, f16 -> f32), numpy single thread"}
    raise ValueError(name)


_start_barrier = None


def _cpu_worker_init(barrier):
    global _start_barrier
    _start_barrier = barrier


def _cpu_worker(job):
    """One process of the parallel oracle baseline: slabs wid, wid + P, ...
    of the same workload until the budget is spent, timed from a barrier
    that every worker reaches after drawing the input."""
    wid, nproc, budget_s = job
    import numpy as np

    import workloads as W
    from oracle import reference as REF

    x, a, b = W.fma_rows_f32((128, 500, 1024), seed=4)
    _start_barrier.wait()
    done, t0 = 0, time.perf_counter()
    while True:
        k = (wid + done * nproc) % 128
        REF.stream_ewise("fma", x[k], a[k], b[k], np.float32)
        done += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return done, el


def cpu_baseline_c4_parallel(budget_s: float):
    """The same oracle over the host's cores: one process per core (at most
    16), each on its own slabs of the workload; aggregate bytes over the
    longest worker's time."""
    import multiprocessing as mp

    nproc = max(1, min(16, len(os.sched_getaffinity(0))))
    ctx = mp.get_context("spawn")
    barrier = ctx.Barrier(nproc)
    with ctx.Pool(nproc, initializer=_cpu_worker_init, initargs=(barrier,)) as pool:
        res = pool.map(_cpu_worker, [(i, nproc, budget_s) for i in range(nproc)])
    done = sum(d for d, _ in res)
    el = max(e for _, e in res)
    nbytes = done * (500 * 1024 * 4 * 2 + 500 * 8)
    return {"value": round(nbytes / el / 1e9, 4), "unit": "GB/s", "cores": nproc, "kind": "oracle",
            "sample": f"{done} [500,1024] f32 slabs of the streamed-fma workload over {nproc} processes "
                      f"in {el:.1f} s, numpy single thread each"}


if __name__ == "__main__":
    main()
