"""bench.py's command line on the CPU host: more than one GPU is refused with
a JSON line that says why, before any GPU work; the argument table parses."""
from __future__ import annotations

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def run_bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = run_bench("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_help_lists_the_options():
    r = run_bench("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--attention", "--pool", "--graph", "--k"):
        assert opt in r.stdout
