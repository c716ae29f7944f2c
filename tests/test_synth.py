"""The seeded input generator: determinism and workload structure (no GPU)."""
from __future__ import annotations

import numpy as np
import pytest

from sparse_attention_kv_qsa_amd import synth


def test_workload_table():
    w = synth.WORKLOADS
    assert [x.name for x in w.values()] == ["tiny-decode", "prompt-32k", "decode-128k",
                                            "prompt-128k", "prompt-256k-tie",
                                            "decode-128k-t2", "decode-128k-t4",
                                            "prompt-128k-shard8"]
    assert [w[n].nq for n in ("decode-128k", "decode-128k-t2", "decode-128k-t4")] == [1, 2, 4]
    assert (w["tiny-decode"].active, w["tiny-decode"].K, w["tiny-decode"].k) == (512, 256, 64)
    assert (w["prompt-32k"].nq, w["prompt-32k"].active, w["prompt-32k"].k) == (256, 8193, 256)
    assert (w["decode-128k"].active, w["decode-128k"].capacity) == (32770, 65538)
    assert (w["prompt-128k"].n_needles, w["prompt-32k"].n_needles) == (328, 82)
    assert w["prompt-256k-tie"].n_needles == 66
    # one of 8 GPUs' share of the 128K prompt's blocks (ranges of 4,096 or 4,097)
    sh = w["prompt-128k-shard8"]
    assert (sh.nq, sh.active, sh.k) == (256, -(-w["prompt-128k"].active // 8), 512)
    # a 262,144-cell capacity is max-context/4 + 2 blocks
    assert w["prompt-128k"].capacity == 262144 // 4 + 2


def test_deterministic_in_seed():
    w = synth.WORKLOADS["tiny-decode"]
    a, b = synth.make_batch(w), synth.make_batch(w)
    assert synth.fingerprint(a.q) == synth.fingerprint(b.q)
    assert synth.fingerprint(a.kblk) == synth.fingerprint(b.kblk)
    c = synth.make_batch(w, seed=1)
    assert synth.fingerprint(a.q) != synth.fingerprint(c.q)


def test_needles_and_poison():
    w = synth.Workload("t", nq=8, heads=2, dim=16, active=500, capacity=520, k=10,
                       needle_frac=0.02, poison=True)
    bt = synth.make_batch(w)
    assert len(bt.needle_blocks) == 10 and len(set(bt.needle_blocks.tolist())) == 10
    assert np.all(np.isnan(bt.kblk[500:])) and np.all(np.isfinite(bt.kblk[:500]))
    for b, j in zip(bt.needle_blocks, bt.needle_queries):
        # a needle is 0.8*q_j + 0.2*noise: strongly aligned with q_j
        x, y = bt.kblk[b].ravel(), bt.q[j].ravel()
        assert np.dot(x, y) / (np.linalg.norm(x) * np.linalg.norm(y)) > 0.9


def test_tie_workload_has_few_distinct_rows():
    w = synth.Workload("t", nq=4, heads=2, dim=8, active=3000, capacity=3000, k=100,
                       needle_frac=0.001, tie_vectors=64)
    bt = synth.make_batch(w)
    distinct = np.unique(bt.kblk.reshape(w.active, -1), axis=0)
    assert len(distinct) <= 64 + w.n_needles


def test_integer_inputs_range():
    q, kb = synth.make_random(3, 4, 8, 20, capacity=24, integer=True)
    assert q.dtype == np.float32 and np.all(np.abs(q) <= 8) and np.all(q == np.round(q))
    assert np.all(np.isnan(kb[20:]))


@pytest.mark.slow
def test_full_workload_shapes():
    bt = synth.make_batch(synth.WORKLOADS["prompt-32k"])
    assert bt.q.shape == (256, 4, 128) and bt.kblk.shape == (8193, 4, 128)
    assert bt.q.dtype == np.float32 and bt.kblk.dtype == np.float32


def test_kv_cache_shapes_and_poison():
    w = synth.Workload("t", nq=1, heads=2, dim=8, active=10, capacity=12, k=4, poison=True)
    kc, vc = synth.make_kv(w)
    assert kc.shape == vc.shape == (48, 2, 8) and kc.dtype == np.float32
    assert np.all(np.isfinite(kc[:40])) and np.all(np.isnan(kc[40:])) and np.all(np.isnan(vc[40:]))
    assert not np.array_equal(kc[:40], vc[:40])
    k2, v2 = synth.make_kv(w)
    assert np.array_equal(kc[:40], k2[:40]) and np.array_equal(vc[:40], v2[:40])


def test_int8_pool():
    codes, scales = synth.make_pool_i8(40, 32, 2, 16, seed=3)
    assert codes.shape == (40, 2, 16) and codes.dtype == np.int8
    assert scales.shape == (40, 2) and scales.dtype == np.uint16
    assert codes.min() >= -127 and codes.max() <= 127 and np.all(codes[32:] == 0)
    s = scales.view(np.float16).astype(np.float64)
    assert np.all((s[:32] >= 0.0099) & (s[:32] <= 0.0401)) and np.all(np.isnan(s[32:]))
    c2, s2 = synth.make_pool_i8(40, 32, 2, 16, seed=3)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
