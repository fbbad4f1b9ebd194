#!/usr/bin/env python3
"""Throughput of the pipelined tile copy + elementwise path on one MI355X.

Default workload: y = a[row] * x + b[row] over a [128, 500, 1024] float32
tensor streamed through a 4-stage LDS ring (stage = two 1024-element rows,
256 threads, one persistent workgroup per CU), the configuration the HBM-roofline target is
quoted on.  One step = one launch of acp_stream_ewise over the whole tensor.
The same line also reports the 2- and 3-stage rings ("ring_stages").  Inputs are seeded synthetic
tensors resident in HBM; three buffer sets are rotated so that consecutive
steps never hit data left in the 256 MB last-level cache by the previous one.

Prints ONE JSON line (rank 0) with the metric, the roofline of the kernel
(its average launch duration from HIP events around the timed region, on the
stream it runs on) and the CPU oracle timed on a bounded sample of the same
workload.

Other workloads (for measurement only): --workload c2 | c3 | c5.
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
                  "acp_k_copy.hip", "acp_api.cpp"]


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


def traffic_from_profiles(workload_key: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", f"{workload_key}.md")
    if not os.path.exists(path):
        return None
    txt = open(path).read()
    m_hash = re.search(r"kernel_source_hash:\s*(\w+)", txt)
    m_bytes = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", txt)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_hash():
        return None
    return float(m_bytes.group(1))


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="c4", choices=["c1", "c2", "c3", "c4", "c5", "calib", "copy_ref", "pointwise", "reduce", "rowsum"],
                    help="c4: the streamed fma (default); c2/c3/c5: the other workloads; "
                         "calib: torch's copy of 256 MiB, the known-size kernel that scales HBM counters; "
                         "copy_ref: the library's register-path reference copy of the c4 tensor "
                         "(the plain 1:1 read/write ceiling)")
    ap.add_argument("--stages", type=int, default=None,
                    help="ring slots (default: the measured best per workload; c4 and c5: 4)")
    ap.add_argument("--z-staging", default="ring", choices=["ring", "set"],
                    help="pointwise: how the second tensor reaches the ring")
    ap.add_argument("--reduce-over-batch", action="store_true",
                    help="reduce: add all 128 slabs into one [500,1024] destination (else slab by slab)")
    ap.add_argument("--rows", type=int, default=None,
                    help="rows per ring stage or tile (default per workload: c4 2, pointwise / reduce / rowsum 4, "
                         "reduce --reduce-over-batch 2)")
    ap.add_argument("--threads", type=int, default=256, help="threads per workgroup")
    ap.add_argument("--workgroups", type=int, default=None,
                    help="persistent workgroups (default 256 x --wg-per-cu; 0: one workgroup per tile)")
    ap.add_argument("--wg-per-cu", type=int, default=1)
    ap.add_argument("--sets", type=int, default=3, help="rotated buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="budget of the oracle sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ring-sweep", action="store_true", help="c4: skip the 2/3-stage report (profiling runs)")
    args = ap.parse_args()
    # defaults: the best launch shapes measured on MI355X for each workload
    wl = args.workload
    if args.rows is None:
        args.rows = {"c4": 2, "pointwise": 4, "rowsum": 4}.get(wl, 2 if args.reduce_over_batch else 4)
    if args.stages is None:
        args.stages = 2 if wl in ("pointwise", "rowsum") else 4
    return args


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build measures one GPU only: every box has one MI355X; "
                                   "run with --gpus 1", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import async_copy_pipelining_amd as acp
    import workloads as W

    dev = "cuda:0"
    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.uint8).reshape(-1).copy()).to(dev)

    def packed(shape):
        st, out = 1, []
        for e in reversed(shape):
            out.append(st)
            st *= e
        return tuple(reversed(out))

    wl = args.workload
    launches = []          # one callable per buffer set
    if wl == "c4":
        shape = (128, 500, 1024)
        stage = (1, args.rows, 1024)
        x, a, b = W.fma_rows_f32(shape, seed=4)
        G = 256 * args.wg_per_cu if args.workgroups is None else args.workgroups
        descs, keep = [], []
        for s in range(args.sets):
            xd, ad, bd = to_dev(x), to_dev(a), to_dev(b)
            yd = torch.empty(x.nbytes, dtype=torch.uint8, device=dev)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, packed(shape), stage)
            ydesc = acp.acp_encode_tiled("f32", yd, shape, packed(shape), stage)
            descs.append((xdesc, ydesc, ad, bd))
            keep.append((xd, yd))
            launches.append((lambda xdesc=xdesc, ydesc=ydesc, ad=ad, bd=bd, keep=(xd, yd):
                             acp.acp_stream_ewise("fma", ydesc, xdesc, ad, bd, stage, args.stages,
                                                  args.threads, G, stream)))
        ring_launches = {st: [(lambda xdesc=xdesc, ydesc=ydesc, ad=ad, bd=bd, st=st:
                               acp.acp_stream_ewise("fma", ydesc, xdesc, ad, bd, stage, st, args.threads, G, stream))
                              for (xdesc, ydesc, ad, bd) in descs] for st in (2, 3, 4)}
        bytes_per = x.nbytes * 2 + a.nbytes + b.nbytes
        dtype = "f32"
        config = {"workload": f"stream fma y=a[row]*x+b[row], [128,500,1024] f32, {args.stages}-stage LDS ring, "
                              f"stage (1,{args.rows},1024)", "shape": list(shape), "stages": args.stages,
                  "stage_box": list(stage), "threads": args.threads, "workgroups": G}
        key = f"stream_fma_f32_128x500x1024_s{args.stages}_r{args.rows}"
    elif wl == "c1":
        # one 8x256 f16 tile through the 128-byte swizzled LDS image and back,
        # 64 threads: latency-bound, so the figure that matters is the launch
        # time (ms_per_step), not the GB/s
        x = W.tile_bits_f16((8, 256), seed=1)
        shape = x.shape
        for s in range(args.sets):
            xd = to_dev(x)
            yd = torch.empty(x.nbytes, dtype=torch.uint8, device=dev)
            xdesc = acp.acp_encode_tiled("f16", xd, shape, packed(shape), shape, acp.ACP_SWIZZLE_128B)
            ydesc = acp.acp_encode_tiled("f16", yd, shape, packed(shape), shape, acp.ACP_SWIZZLE_128B)
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_tile_copy(xdesc, ydesc, 64, stream))
        bytes_per, dtype = x.nbytes * 2, "f16"
        config = {"workload": "swizzled tile copy, one 8x256 f16 tile (128-byte swizzle), 64 threads "
                              "(latency-bound: read ms_per_step)"}
        key = "tile_copy_f16_8x256_swizzle128"
    elif wl == "c2":
        x = W.sqrt_tiles_f32(65536, seed=2)
        shape = x.shape
        for s in range(args.sets):
            xd = to_dev(x)
            yd = torch.empty(x.nbytes, dtype=torch.uint8, device=dev)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, packed(shape), (1, 32, 32))
            ydesc = acp.acp_encode_tiled("f32", yd, shape, packed(shape), (1, 32, 32))
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_tile_ewise("sqrt", ydesc, [xdesc], 256, stream))
        bytes_per, dtype = x.nbytes * 2, "f32"
        config = {"workload": "tile sqrt, 65536 tiles of 32x32 f32, 256 threads, persistent grid"}
        key = "tile_sqrt_f32_65536x32x32"
    elif wl == "c3":
        shape = (128, 500, 1024)
        x = W.normal_f16(shape, seed=3)
        for s in range(args.sets):
            xd = to_dev(x)
            yd = torch.empty(x.nbytes, dtype=torch.uint8, device=dev)
            xdesc = acp.acp_encode_tiled("f16", xd, shape, packed(shape), (1, 128, 32))
            ydesc = acp.acp_encode_tiled("f16", yd, shape, packed(shape), (1, 128, 32))
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_tile_copy(xdesc, ydesc, 128, stream))
        bytes_per, dtype = x.nbytes * 2, "f16"
        config = {"workload": "tile copy, [128,500,1024] f16, 128x32 tiles, 128 threads"}
        key = "tile_copy_f16_128x500x1024"
    elif wl == "pointwise":
        # y = x + z over two [128,500,1024] f32 tensors, both streamed
        shape = (128, 500, 1024)
        stage = (1, args.rows, 1024)
        rng = np.random.default_rng(6)
        x = rng.standard_normal(shape, dtype=np.float32)
        z = rng.standard_normal(shape, dtype=np.float32)
        G = 256 * args.wg_per_cu if args.workgroups is None else args.workgroups
        for s in range(args.sets):
            xd, zd = to_dev(x), to_dev(z)
            yd = torch.empty(x.nbytes, dtype=torch.uint8, device=dev)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, packed(shape), stage)
            zdesc = acp.acp_encode_tiled("f32", zd, shape, packed(shape), stage)
            ydesc = acp.acp_encode_tiled("f32", yd, shape, packed(shape), stage)
            launches.append(lambda xdesc=xdesc, zdesc=zdesc, ydesc=ydesc, keep=(xd, zd, yd):
                            acp.acp_stream_binary("add", ydesc, xdesc, zdesc, stage, args.stages, args.threads, G,
                                                  args.z_staging, stream))
        bytes_per, dtype = 3 * x.nbytes, "f32"
        config = {"workload": f"two-tensor stream y = x + z, [128,500,1024] f32, {args.stages}-stage LDS ring, "
                              f"stage (1,{args.rows},1024), z staged '{args.z_staging}'", "workgroups": G}
        key = f"stream_add2_f32_128x500x1024_s{args.stages}_r{args.rows}_{args.z_staging}"
    elif wl == "reduce":
        # store with reduce-add of a [128,500,1024] f32 tensor in (1,R,1024)
        # tiles: into a same-shape destination (one contribution per element)
        # or into one [1,500,1024] slab (128 contributions per element)
        shape = (128, 500, 1024)
        dshape = (1, 500, 1024) if args.reduce_over_batch else shape
        box = (1, args.rows, 1024)
        rng = np.random.default_rng(7)
        x = rng.standard_normal(shape, dtype=np.float32)
        for s in range(args.sets):
            xd = to_dev(x)
            yd = torch.zeros(int(np.prod(dshape)) * 4, dtype=torch.uint8, device=dev)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, packed(shape), box)
            ydesc = acp.acp_encode_tiled("f32", yd, dshape, packed(dshape), box)
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_tile_reduce("add", ydesc, xdesc, args.threads, stream))
        # algorithmic bytes: the source once, the destination read and written once
        bytes_per, dtype = x.nbytes + 2 * int(np.prod(dshape)) * 4, "f32"
        config = {"workload": f"store with reduce-add, [128,500,1024] f32 tiles (1,{args.rows},1024) into "
                              f"{list(dshape)}"}
        key = f"tile_reduce_f32_128x500x1024_r{args.rows}_{'batch' if args.reduce_over_batch else 'slab'}"
    elif wl == "rowsum":
        # y[i, j] = sum over k of x[i, j, k], [128,500,1024] f32 -> [128,500]
        shape = (128, 500, 1024)
        stage = (1, args.rows, 1024)
        rng = np.random.default_rng(8)
        x = rng.standard_normal(shape, dtype=np.float32)
        G = 256 * args.wg_per_cu if args.workgroups is None else args.workgroups
        for s in range(args.sets):
            xd = to_dev(x)
            yd = torch.empty(128 * 500 * 4, dtype=torch.uint8, device=dev)
            xdesc = acp.acp_encode_tiled("f32", xd, shape, packed(shape), stage)
            launches.append(lambda xdesc=xdesc, keep=(xd, yd):
                            acp.acp_stream_reduce_rows("add", keep[1], xdesc, stage, args.stages, args.threads, G,
                                                       stream))
        bytes_per, dtype = x.nbytes + 128 * 500 * 4, "f32"
        config = {"workload": f"row sums of [128,500,1024] f32 -> [128,500], {args.stages}-stage LDS ring, "
                              f"stage (1,{args.rows},1024)", "workgroups": G}
        key = f"stream_rowsum_f32_128x500x1024_s{args.stages}_r{args.rows}"
    elif wl == "copy_ref":
        n = 128 * 500 * 1024 * 4
        G = 256 * args.wg_per_cu if args.workgroups is None else args.workgroups
        for s in range(args.sets):
            xd = torch.ones(n, dtype=torch.uint8, device=dev)
            yd = torch.empty(n, dtype=torch.uint8, device=dev)
            launches.append(lambda xd=xd, yd=yd: acp.acp_debug_stream_copy(yd, xd, n, G, stream))
        bytes_per, dtype = 2 * n, "u8"
        config = {"workload": f"reference register-path copy of 262144000 B (the c4 tensor), {G} workgroups"}
        key = "stream_copy_reference_262MB"
    elif wl == "calib":
        n = 256 << 20
        for s in range(args.sets):
            xd = torch.ones(n, dtype=torch.uint8, device=dev)
            yd = torch.empty(n, dtype=torch.uint8, device=dev)
            launches.append(lambda xd=xd, yd=yd: yd.copy_(xd))
        bytes_per, dtype = 2 * n, "u8"
        config = {"workload": "torch copy_ of 256 MiB (counter calibration: 268435456 B read, 268435456 B written)"}
        key = "calib_copy_256MiB"
    else:
        shape, pitch = (4, 8, 64, 128, 256), 264
        storage, strides = W.padded_uniform_f16(shape, pitch=pitch, seed=5)
        n = int(np.prod(shape))
        for s in range(args.sets):
            xd = to_dev(storage)
            yd = torch.empty(n * 4, dtype=torch.uint8, device=dev)
            xdesc = acp.acp_encode_tiled("f16", xd, shape, strides, (1, 2, 16, 64, 64), acp.ACP_SWIZZLE_128B)
            ydesc = acp.acp_encode_tiled("f32", yd, shape, packed(shape), (1, 2, 16, 64, 64))
            launches.append(lambda xdesc=xdesc, ydesc=ydesc, keep=(xd, yd):
                            acp.acp_stream_ewise("exp", ydesc, xdesc, None, None, (1, 1, 1, 64, 64),
                                                 args.stages, 256, 0, stream))
        bytes_per, dtype = n * 2 + n * 4, "f16->f32"
        config = {"workload": "rank-5 exp (4,8,64,128,256) f16 pitch 264 -> f32, box (1,2,16,64,64), "
                              f"{args.stages}-stage swizzled ring, stage (1,1,1,64,64)"}
        key = f"stream_exp_rank5_s{args.stages}"

    for i in range(args.warmup):
        launches[i % len(launches)]()
    torch.cuda.synchronize()
    kernel = acp.acp_last_kernel()          # the launch shape the library chose for the timed kernel
    if kernel:
        config = {**config, "kernel": kernel}

    # Timed region: K steps back to back, bracketed by synchronize and one
    # event pair on the launch stream.
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(args.steps):
        launches[i % len(launches)]()
    t1.record(stream)
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)

    # One step is one launch of the kernel, on the stream the events were
    # recorded on: the timed region's events give its average launch
    # duration (the figure rocprofv3's kernel trace reports per dispatch).
    ms_per_step = total_ms / args.steps
    avg_launch_ms = ms_per_step
    value = bytes_per / (ms_per_step * 1e-3) / 1e9
    achieved = bytes_per / (avg_launch_ms * 1e-3) / 1e9

    # For reference: the same K launches, each bracketed by its own event
    # pair (this adds the dispatch gap to every launch).
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    for i in range(args.steps):
        starts[i].record(stream)
        launches[i % len(launches)]()
        ends[i].record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(s.elapsed_time(e) for s, e in zip(starts, ends))

    ring = None
    if wl == "c4" and not args.no_ring_sweep:
        # the 2-, 3- and 4-stage rings, back to back like `value`
        ring = {}
        for st in (2, 3, 4):
            fns = ring_launches[st] if st != args.stages else launches
            for i in range(args.warmup):
                fns[i % len(fns)]()
            torch.cuda.synchronize()
            r0 = torch.cuda.Event(enable_timing=True)
            r1 = torch.cuda.Event(enable_timing=True)
            r0.record(stream)
            for i in range(args.steps):
                fns[i % len(fns)]()
            r1.record(stream)
            torch.cuda.synchronize()
            ring[str(st)] = round(bytes_per / (r0.elapsed_time(r1) / args.steps * 1e-3) / 1e9, 1)

    traffic = traffic_from_profiles(key)
    result = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
        "data": "synthetic (seeded numpy draws resident in HBM, 3 rotated buffer sets)",
        "config": config,
        "percent_of_peak": round(100.0 * value / PEAK_GBS, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_GBS, 4), "traffic": traffic,
                     "algorithmic_bytes_per_launch": bytes_per,
                     "avg_launch_ms": round(avg_launch_ms, 5),
                     "median_event_bracketed_launch_ms": round(per_launch[len(per_launch) // 2], 5),
                     "kernel_source_hash": kernel_hash()},
    }
    if ring is not None:
        result["ring_stages"] = {"unit": "GB/s", **ring}
    if not args.no_cpu_baseline and wl == "c4":
        result["cpu_baseline"] = cpu_baseline_c4(args.cpu_seconds)
        result["cpu_baseline_all_cores"] = cpu_baseline_c4_parallel(args.cpu_seconds)
    print(json.dumps(result), flush=True)


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
    import os

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
