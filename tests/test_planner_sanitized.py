"""The C++ planner (acp_plan.cpp, host code with no HIP) on random
descriptors, built with g++ and the address and undefined-behaviour
sanitizers: no out-of-bounds access, overflow or other undefined behaviour
on any accepted, declined or unsupported request."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "async_copy_pipelining_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_planner_under_sanitizers(tmp_path):
    exe = str(tmp_path / "planner_fuzz")
    flags = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
    subprocess.run(["g++", "-std=c++17", "-O1", "-g", *flags, f"-I{CSRC}", "-o", exe,
                    os.path.join(ROOT, "tests", "planner_fuzz.cpp"), os.path.join(CSRC, "acp_plan.cpp")],
                   check=True, capture_output=True, timeout=300)
    r = subprocess.run([exe, "100000"], capture_output=True, text=True, timeout=300,
                       env={**os.environ, "ASAN_OPTIONS": "detect_leaks=1"})
    assert r.returncode == 0, r.stderr[-2000:]
    counts = dict(zip(r.stdout.split()[::2], map(int, r.stdout.split()[1::2])))
    assert counts["ok"] > 1000 and counts["declined"] > 0 and counts["unsupported"] > 0, r.stdout
    assert counts["ok"] + counts["declined"] + counts["unsupported"] + counts["invalid"] == 100000
