"""bench.py without a GPU: the one-GPU contract and the rocprofv3 summaries it
reads its HBM traffic from."""
import json
import os
import re
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=60)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_profile_summaries_name_their_commands_and_kernel_sources():
    names = sorted(f for f in os.listdir(PROFILES) if f.endswith(".md"))
    assert names
    for name in names:
        text = open(os.path.join(PROFILES, name), encoding="utf-8").read()
        assert re.search(r"^kernel_source_hash: [0-9a-f]{16}$", text, re.M), name
        # a profiled run (optionally with the row's environment exported
        # first), or the plain default bench run whose line a summary records
        cmds = re.findall(r"^\s+(?:<env> )?rocprofv3 .* -- python3 \$R/bench\.py .*$", text, re.M)
        plain = re.findall(r"^\s+python3 \$R/bench\.py.*$", text, re.M)
        assert cmds or plain, name
        for c in cmds + plain:
            # only committed files run: the bench itself, no helper scripts
            assert "_work" not in c, c
        for c in cmds:
            assert re.search(r" -d \$R/\S+ ", c), c       # output under the repository root


def test_headline_profile_matches_the_bench_default():
    # the default workload (streamed fma, 4 slots, stage (1,2,1024)) reads its
    # traffic from this summary
    src = open(os.path.join(ROOT, "bench.py"), encoding="utf-8").read()
    c4 = src[src.index('if name == "c4":'):src.index('elif name == "c1":')]
    assert "rows = args.rows or 2" in c4 and "S = stages or args.stages or 4" in c4
    assert os.path.exists(os.path.join(PROFILES, "stream_fma_f32_128x500x1024_s4_r2.md"))
