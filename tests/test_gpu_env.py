"""GPU parity of the linear-grid kernels with cached loads and stores.

Non-temporal loads and stores (the default for contiguous stages) run a
kernel body whose cache policy is fixed at compile time; with either turned
off (ACP_LOAD_NT=0, ACP_STORE_NT=0) the body that takes the policy at run
time runs instead.  The library reads these knobs once per process, so the
cases run in one child process (tests/gpu_env_child.py) that checks every
result against the oracle."""
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))


def test_linear_kernels_with_cached_loads_and_stores():
    env = dict(os.environ, ACP_LOAD_NT="0", ACP_STORE_NT="0")
    print("[gpu] child process: linear kernels with ACP_LOAD_NT=0 ACP_STORE_NT=0", flush=True)
    r = subprocess.run([sys.executable, "-u", os.path.join(HERE, "gpu_env_child.py")], env=env,
                       capture_output=True, text=True, timeout=110)
    print(r.stdout[-3000:], flush=True)
    assert r.returncode == 0, r.stderr[-3000:]
    assert "all ok" in r.stdout
