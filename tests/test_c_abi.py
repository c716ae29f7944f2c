"""The C ABI from plain C: tests/c_abi/select_attend.c includes only
include/qsa.h and the HIP runtime's C API.  On the CPU it must compile as
C11 with every warning as an error and link against libqsa.so; on the GPU
its select + attention results must meet the same gates as the Python
binding's (scores within 1e-6 of max|s| of FP64, ids equal to the oracle's
selection on the GPU's scores, attention within the derived gate)."""
from __future__ import annotations

import os
import subprocess
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "c_abi"))

import build_example as c_build  # noqa: E402  (tests/c_abi/build_example.py)
import oracle  # noqa: E402
from checks import attn_limit, score_gate  # noqa: E402
from sparse_attention_kv_qsa_amd import binding, synth  # noqa: E402


def test_c_program_compiles_against_the_header(tmp_path):
    if not os.path.exists(binding.library_path()):
        pytest.fail("libqsa.so is not built (run __graft_entry__.build())")
    exe = c_build.build(out=str(tmp_path / "select_attend"))
    assert os.path.getsize(exe) > 0


@pytest.mark.gpu
@pytest.mark.parametrize("nq,heads,dim,active,capacity,k", [
    (1, 4, 64, 512, 512, 64), (4, 4, 128, 3000, 3002, 200), (2, 2, 32, 70, 80, 100)])
def test_c_program_matches_the_oracle(tmp_path, nq, heads, dim, active, capacity, k):
    exe = c_build.EXE
    if not os.path.exists(exe):  # a gcc link of one small file, on the host
        c_build.build()
    q, kb = synth.make_random(nq, heads, dim, active, capacity=capacity, seed=active + k)
    w = synth.Workload("c", nq=nq, heads=heads, dim=dim, active=active, capacity=capacity, k=k,
                       poison=True)
    kc, vc = synth.make_kv(w, seed=3)
    for name, a in (("q", q), ("kblk", kb), ("kc", kc), ("vc", vc)):
        np.ascontiguousarray(a, np.float32).tofile(tmp_path / f"{name}.bin")
    r = subprocess.run([exe, str(tmp_path), str(nq), str(heads), str(dim), str(active),
                        str(capacity), str(k)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    s = np.fromfile(tmp_path / "scores.bin", np.float32).reshape(nq, active)
    ids = np.fromfile(tmp_path / "ids.bin", np.int32).reshape(nq, k)
    out = np.fromfile(tmp_path / "out.bin", np.float32).reshape(nq, heads, dim)
    ok, ratio = score_gate(s, oracle.scores_f64(q, kb, active))
    assert ok, f"score error {ratio:.2f}x the gate"
    assert np.array_equal(ids, oracle.topk(s, k))
    scale = 1.0 / np.sqrt(dim)
    o64 = oracle.sparse_decode_attn_f64(q, kc, vc, ids, 4 * active, scale)
    err = np.abs(out.astype(np.float64) - o64).max(axis=2)
    assert np.all(err <= attn_limit(q, kc, vc, ids, 4 * active, scale))
