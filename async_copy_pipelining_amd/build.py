"""Build ``libacp.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python async_copy_pipelining_amd/build.py`` (run as a script: importing
the package needs the library it builds), or ``__graft_entry__.build()``.  Always
recompiles.  Device code is built with packed-fp32 instructions disabled and
without fast-math, so fp32 results keep IEEE rounding and denormals.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libacp.so")
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall", "-Wno-unused-function"]
DEVICE = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-fno-gpu-rdc"]

SOURCES = [
    ("acp_plan.cpp", False),
    ("acp_api.cpp", False),
    ("acp_engine.hip", True),
    ("acp_k_copy.hip", True),
    ("acp_k_tile.hip", True),
    ("acp_k_tile_gen.hip", True),
    ("acp_k_tile_lin.hip", True),
    ("acp_k_stream_f32.hip", True),
    ("acp_k_stream_f16.hip", True),
    ("acp_k_ref.hip", True),
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}")
    return r


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cmds, objs = [], []
    for src, device in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmds.append([HIPCC] + COMMON + (DEVICE + ["-x", "hip"] if device else []) +
                    ["-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    if verbose:
        for c in cmds:
            print(" ".join(c))
    jobs = jobs or min(len(cmds), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(_run, cmds))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd))
    _run(cmd)
    shutil.move(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
