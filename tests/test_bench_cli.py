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


def test_cpu_baseline_reports_stages_and_threads():
    """The CPU-baseline leg on the tiny decode workload: all-core and
    single-thread runs, scores and top-k timed apart."""
    sys.path.insert(0, ROOT)
    import bench
    from sparse_attention_kv_qsa_amd import synth

    w = synth.WORKLOADS["tiny-decode"]
    out = bench.cpu_baseline(w, synth.make_batch(w))
    assert out["kind"] == "oracle" and out["unit"] == bench.UNIT
    assert 1 <= out["cores"] <= out["affinity_cores"]
    for leg in (out, out["single_thread"]):
        assert leg["value"] > 0 and leg["scores_value"] > 0 and leg["topk_value"] > 0
        # the combined rate is the harmonic combination of the two steps
        both = 1.0 / (1.0 / leg["scores_value"] + 1.0 / leg["topk_value"])
        assert abs(leg["value"] - both) <= 1e-6 * both
    assert out["single_thread"]["cores"] == 1


def test_spread_and_select_bytes():
    sys.path.insert(0, ROOT)
    import bench
    from sparse_attention_kv_qsa_amd import synth

    sp = bench.spread([3.0, 1.0, 2.0])
    assert sp == {"n": 3, "median_ms": 2.0, "min_ms": 1.0, "max_ms": 3.0}
    w = synth.WORKLOADS["decode-128k"]
    # summaries 32,770 x 512 floats, one query, scores written and read, 512 ids
    assert bench.select_bytes(w) == 4.0 * (32770 * 512 + 512 + 2 * 32770 + 512)
