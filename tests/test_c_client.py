"""The C ABI from plain C: tests/c_client.c compiles as C99 with -pedantic
against include/acp.h, links libacp.so and runs its host-only calls."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PKG = os.path.join(ROOT, "async_copy_pipelining_amd")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_plain_c_client(tmp_path):
    exe = tmp_path / "c_client"
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", f"-I{os.path.join(ROOT, 'include')}",
           os.path.join(ROOT, "tests", "c_client.c"), "-o", str(exe), f"-L{PKG}", "-lacp", f"-Wl,-rpath,{PKG}"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stdout + out.stderr
    lines = out.stdout.splitlines()
    # the worked example's descriptor: rank 3, dims (64, 8, 4), strides (512, 128) bytes, box (64, 8, 4)
    assert lines[0] == "rank 3 dims 64 8 4 strides 2 512 128 box 64 8 4 vec 8 vec_bytes 16 outer 4"
    assert lines[1] == "declined 1 innermost stride must be 1"
    assert lines[2] == "abi 1"
