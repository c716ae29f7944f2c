"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Gates (identical at every size):
* scores: max |s_gpu - s64| <= 1e-6 * max |s64| over the call (s64 = FP64 oracle);
  bitwise equality wherever the exact result is an fp32 number (hand example,
  small-integer inputs);
* ids: bit-exact against the oracle's sort-based top-k applied to the GPU's
  own fp32 scores.
At the full workload sizes the FP64 scores of every query row are computed
(rows over host threads) and top-k is checked on every row; the margins (the
error against the gate over the call and per row, and the agreement of the
selection with the selection on the FP64 scores) are printed and, with
QSA_MARGINS_DIR set, written there as JSON.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import pytest

import oracle
from checks import SCORE_TOL, score_gate, topk_invariants
from sparse_attention_kv_qsa_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

ORC = oracle.default()


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_kv_qsa_amd import binding
    lib = binding.load_library()
    assert binding.library_path().startswith(os.path.dirname(os.path.dirname(__file__)))
    return lib


MODES = ["fp32", "bf16x3", "f16x2"]  # "auto" is one of these for every shape


def gpu_scores(q: np.ndarray, kblk: np.ndarray, active: int, mode="auto") -> np.ndarray:
    from sparse_attention_kv_qsa_amd import qsa_block_scores_ex
    s = qsa_block_scores_ex(torch.from_numpy(q).cuda(), torch.from_numpy(kblk).cuda(), active,
                            mode=mode)
    torch.cuda.synchronize()
    return s.cpu().numpy()


def gpu_topk(scores: np.ndarray, k: int) -> np.ndarray:
    from sparse_attention_kv_qsa_amd import qsa_block_topk
    ids = qsa_block_topk(torch.from_numpy(np.ascontiguousarray(scores, np.float32)).cuda(), k)
    torch.cuda.synchronize()
    return ids.cpu().numpy()


def check_scores(s, s64):
    ok, ratio = score_gate(s, s64, SCORE_TOL)
    assert ok, f"score error {ratio:.3f}x the gate"
    return ratio


FEW_ROWS = 16  # QSA_TOPK_FEW_ROWS: batches up to this many rows take the whole-GPU path
PATHS = ["few-rows", "per-row"]


def rows_for_path(scores: np.ndarray, path: str) -> np.ndarray:
    """The same rows as a batch that takes the given top-k path: at most
    FEW_ROWS rows for the whole-GPU path, more than that (the rows repeated)
    for the one-workgroup-per-row path."""
    if path == "few-rows":
        assert scores.shape[0] <= FEW_ROWS
        return scores
    reps = FEW_ROWS // scores.shape[0] + 1
    return np.ascontiguousarray(np.tile(scores, (reps, 1)))


def check_topk(scores, k, path="few-rows"):
    scores = rows_for_path(np.ascontiguousarray(scores, np.float32), path)
    ids = gpu_topk(scores, k)
    want = ORC.topk(scores, k)
    if not np.array_equal(ids, want):
        bad = np.nonzero(np.any(ids != want, axis=1))[0]
        i = bad[0]
        r = np.nonzero(ids[i] != want[i])[0][0]
        raise AssertionError(f"{len(bad)} rows differ; row {i} rank {r}: gpu {ids[i, r]} "
                             f"oracle {want[i, r]} (A={scores.shape[1]}, k={k})")
    return ids


# ------------------------------------------------------------ scores ----

@pytest.mark.parametrize("mode", ["auto"] + MODES)
def test_hand_example_bitwise(mode):
    from test_oracle import load_hand_example
    q, b, scores, topks = load_hand_example()
    want = np.array([scores[i] for i in sorted(scores)], np.float32)
    for reps in (1, 9):  # nq = 2 takes the dot-product kernel, nq = 18 the MFMA tiles
        qq = np.ascontiguousarray(np.tile(q, (reps, 1, 1)))
        s = gpu_scores(qq, b, 3, mode)
        assert np.array_equal(s, np.tile(want, (reps, 1)))
    for i, k, ids in topks:
        assert gpu_topk(want[i:i + 1], k)[0].tolist() == ids


INT_CASES = [  # nq, heads, dim, active (ragged tails against 16/64-wide tiles)
    (1, 4, 64, 512), (1, 1, 4, 1), (3, 3, 4, 77), (8, 4, 128, 130),
    (9, 4, 128, 65), (64, 4, 128, 64), (100, 2, 6, 17), (130, 4, 128, 1000),
    (256, 4, 128, 4097), (17, 1, 132, 300), (70, 4, 16, 129), (1, 8, 64, 33),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("nq,heads,dim,active", INT_CASES)
def test_integer_inputs_bitwise(nq, heads, dim, active, mode):
    q, kb = synth.make_random(nq, heads, dim, active, capacity=active + 5, seed=nq + active,
                              integer=True)
    s = gpu_scores(q, kb, active, mode)
    s64 = ORC.scores_f64(q, kb, active)
    assert np.array_equal(s.astype(np.float64), s64)


RAND_CASES = [  # nq, heads, dim, active
    (1, 4, 64, 512), (1, 4, 128, 3000), (2, 4, 128, 999), (5, 2, 96, 1234), (8, 4, 128, 777),
    (1, 16, 256, 300), (2, 8, 256, 200), (4, 4, 256, 100), (8, 2, 256, 50),
    (9, 4, 128, 1025), (33, 4, 64, 2000), (64, 4, 128, 4096), (256, 4, 128, 2113),
    (200, 4, 100, 515), (16, 32, 128, 70), (40, 1, 4, 333), (12, 3, 20, 64),
    # wide ragged columns (33..63 blocks) with LDS-staged query rows
    (130, 4, 128, 1000), (150, 4, 64, 2047),
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("nq,heads,dim,active", RAND_CASES)
def test_scores_within_gate(nq, heads, dim, active, mode):
    q, kb = synth.make_random(nq, heads, dim, active, capacity=active + 3, seed=7 * nq + dim)
    s = gpu_scores(q, kb, active, mode)
    assert np.all(np.isfinite(s)), "poisoned capacity rows were read"
    check_scores(s, ORC.scores_f64(q, kb, active))


@pytest.mark.parametrize("mode", MODES)
def test_scores_deterministic_and_position_invariant(mode):
    rng = np.random.default_rng(12)
    # 700 blocks end in a 60-block ragged column, 705 in a 1-block one (the
    # split-K ragged path of the bf16 scorer)
    for nq, a in ((1, 700), (5, 705), (100, 700), (300, 700), (300, 705), (70, 705)):
        vec = rng.standard_normal((4, 4, 128)).astype(np.float32)
        assign = rng.integers(0, 4, a)
        kb = np.ascontiguousarray(vec[assign])
        q = rng.standard_normal((nq, 4, 128)).astype(np.float32)
        s1, s2 = gpu_scores(q, kb, a, mode), gpu_scores(q, kb, a, mode)
        assert np.array_equal(s1, s2)
        for c in range(4):
            cols = s1[:, assign == c]
            assert np.all(cols == cols[:, :1]), "identical summaries scored differently"


def test_f16x2_power_of_two_scaling_exact():
    """The fp16 split scales every row by a power of two fixed by the row's
    own data, so scaling a query or a block summary by 2^a scales its scores
    by exactly 2^a (no result near the subnormal or overflow range here),
    whatever the magnitude: rows at 2^-100 and 2^90 score like unit rows."""
    rng = np.random.default_rng(21)
    nq, a = 130, 197  # a ragged query tile and a narrow ragged column (197 % 64 = 5)
    q = rng.standard_normal((nq, 4, 128)).astype(np.float32)
    kb = rng.standard_normal((a, 4, 128)).astype(np.float32)
    s = gpu_scores(q, kb, a, "f16x2")
    check_scores(s, ORC.scores_f64(q, kb, a))
    eq = rng.integers(-60, 60, nq)
    eb = rng.integers(-60, 40, a)
    eq[:3], eb[:3] = (-100, 90, 0), (0, -100, 88)
    q2 = np.ascontiguousarray(np.ldexp(q, eq[:, None, None]).astype(np.float32))
    kb2 = np.ascontiguousarray(np.ldexp(kb, eb[:, None, None]).astype(np.float32))
    ok = np.abs(eq[:, None] + eb[None, :]) < 100  # products stay normal fp32 numbers
    s2 = gpu_scores(q2, kb2, a, "f16x2")
    want = np.ldexp(s.astype(np.float64), eq[:, None] + eb[None, :])
    assert np.array_equal(s2[ok].astype(np.float64), want[ok])


@pytest.mark.parametrize("heads,dim", [(4, 128), (3, 20)])  # K = 512 (LDS-staged queries), 60
def test_f16x2_range_fallback(heads, dim):
    """Rows with an element more than 2^7 times their first-step maximum
    would overflow a binary16 piece: their scores are computed from the two
    rows in FP64 (one rounding), identical wherever the block sits; rows
    whose first step is all zeros stay unscaled; a non-finite input gives
    non-finite scores in its row and column only."""
    rng = np.random.default_rng(22)
    nq, a = 140, 300
    q = rng.standard_normal((nq, heads, dim)).astype(np.float32)
    kb = rng.standard_normal((a, heads, dim)).astype(np.float32)
    kb[3, 2, 5] = 3.0e5          # block 3: far above its first 32 elements
    kb[299] = kb[3]              # the same summary in the narrow ragged column
    kb[64] = kb[3]               # ... and in another full tile
    q[7, -1, -3] = -2.0e6        # query 7 likewise
    q[135] = q[7]                # a copy in the ragged query tile
    kb[10].reshape(-1)[:32] = 0.0  # first step all zeros: unscaled
    kb[11, :, :] = 0.0
    kb[11, -1, -1] = 5.0e4
    s = gpu_scores(q, kb, a, "f16x2")
    s64 = ORC.scores_f64(q, kb, a)
    assert np.all(np.isfinite(s))
    for c in (3, 64, 299):
        assert np.array_equal(s[:, c], s[:, 3])
    assert np.array_equal(s[7], s[135])
    # the fallback's scores: FP64 sum rounded once
    fb = np.zeros(s.shape, bool)
    fb[:, [3, 64, 299]] = True
    fb[[7, 135], :] = True
    assert np.all(np.abs(s[fb] - s64[fb]) <= np.spacing(np.abs(s[fb]).astype(np.float32)))
    # the other rows and columns within the gate on their own
    rows = np.setdiff1d(np.arange(nq), [7, 135])
    cols = np.setdiff1d(np.arange(a), [3, 64, 299])
    check_scores(s[np.ix_(rows, cols)], s64[np.ix_(rows, cols)])
    q3 = q.copy()
    q3[5, 1, 7] = np.inf
    s3 = gpu_scores(q3, kb, a, "f16x2")
    assert not np.any(np.isfinite(s3[5]))
    others = np.arange(nq) != 5
    assert np.array_equal(s3[others], s[others])


def test_scores_canary_untouched(gpu):
    nq, heads, dim, a = 70, 4, 128, 1000
    q, kb = synth.make_random(nq, heads, dim, a, seed=3)
    qt, kt = torch.from_numpy(q).cuda(), torch.from_numpy(kb).cuda()
    out = torch.full((nq * a + 4096,), 12345.0, dtype=torch.float32, device="cuda")
    st = gpu.qsa_block_scores(qt.data_ptr(), kt.data_ptr(), nq, heads, dim, a, out.data_ptr(),
                              torch.cuda.current_stream().cuda_stream or None)
    assert st == 0
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert np.all(o[nq * a:] == 12345.0)
    check_scores(o[: nq * a].reshape(nq, a), ORC.scores_f64(q, kb, a))


# ------------------------------------------------------------- top-k ----

def tie_rows(rng, nq, a, nvals):
    vals = rng.standard_normal(nvals).astype(np.float32)
    return np.ascontiguousarray(vals[rng.integers(0, nvals, (nq, a))])


# (A, k) pairs that straddle every register width (reach (PER+1)*1024) and the
# streaming fallback past 66,560 blocks.
WIDTH_CASES = [
    (1, 1), (2, 1), (17, 5), (512, 64), (1023, 100), (1024, 1024), (1025, 1),
    (2048, 300), (2049, 2048), (4096, 4095), (4097, 512), (8193, 256), (16385, 700),
    (24577, 1000), (32770, 512), (33792, 33), (33793, 4096), (49153, 999), (65538, 1024),
    (66560, 2), (66561, 300), (100003, 1024), (32770, 4096), (32770, 2049),
]


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("a,k", WIDTH_CASES)
def test_topk_widths_random(a, k, path):
    rng = np.random.default_rng(a + k)
    s = (rng.standard_normal((3, a)) * 20).astype(np.float32)
    check_topk(s, k, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("a,k", WIDTH_CASES)
def test_topk_widths_heavy_ties(a, k, path):
    rng = np.random.default_rng(a * 3 + k)
    check_topk(tie_rows(rng, 2, a, 7), k, path)


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("a,k", [(10, 20), (1, 4096), (513, 600), (4000, 4096), (3, 4)])
def test_topk_k_larger_than_row(a, k, path):
    rng = np.random.default_rng(a)
    ids = check_topk(tie_rows(rng, 2, a, 5), k, path)
    assert np.all(ids[:, a:] == -1)


@pytest.mark.parametrize("a,k", [(131072, 1024), (131073, 1024), (65538, 100), (4097, 2000)])
def test_topk_tie_at_threshold(a, k):
    """Rows whose k-th key is shared by many more elements than are still
    needed (a tie at the threshold, resolved by id): rows of up to 131,072
    blocks take the ids through a bitmap of the tied ids, longer ones through
    radix passes over the id; both must give the lowest ids of the tie."""
    rng = np.random.default_rng(a + k)
    s = tie_rows(rng, 3, a, 40)
    s[:, rng.choice(a, 37, replace=False)] = np.float32(50.0)  # a few distinct leaders
    ids = check_topk(s, k, "per-row")
    assert ids.shape[1] == k


def clustered_rows(rng, a):
    """Rows whose best scores crowd into a few places: the whole-GPU path's
    groups holding more winners than they publish (re-read from the scores),
    groups with nothing to offer, and ties at its bound."""
    base = (rng.standard_normal(a) * 5).astype(np.float32)
    rows = []
    r = base.copy(); r[300:1100] += 100                       # one region holds every winner
    rows.append(r)
    r = base.copy(); r[::97] += 60; r[a // 2: a // 2 + 700] += 80   # sparse spikes + a block
    rows.append(r)
    rows.append(np.sort(base))                                # increasing: the tail wins
    rows.append(np.sort(base)[::-1].copy())                   # decreasing: the head wins
    r = np.round(base).astype(np.float32)                     # integers: thousands of ties
    rows.append(r)
    r = base.copy(); r[-3:] = 1e30                            # winners in the ragged last group
    rows.append(r)
    return np.ascontiguousarray(np.stack(rows).astype(np.float32))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("a,k", [(1200, 64), (8193, 256), (32770, 512), (65538, 1024),
                                  (100003, 2048), (5000, 4096)])
def test_topk_clustered(a, k, path):
    rng = np.random.default_rng(a)
    ids = check_topk(clustered_rows(rng, a), k, path)
    assert ids.shape[1] == k


# Long rows on the few-row path: groups of 256 elements (rows of 131,073 to
# 524,288 blocks) and of 1,024 (524,289 to 2,097,152), and past that the
# streaming one-workgroup path.  Heavy-tie rows make nearly every group
# "rich" (more than 1,024 of them at these lengths), so the exact
# one-workgroup fallback runs from the grouped launch as well.
LONG_CASES = [(131073, 64), (300000, 512), (524288, 4096), (524289, 64), (600000, 1024),
              (2000000, 4096), (2097152, 300), (2097153, 512)]


@pytest.mark.slow
@pytest.mark.parametrize("a,k", LONG_CASES)
def test_topk_long_rows(a, k):
    rng = np.random.default_rng(a + 7 * k)
    print(f"\n[long rows] A={a} k={k}", flush=True)
    check_topk((rng.standard_normal((2, a)) * 20).astype(np.float32), k)
    check_topk(tie_rows(rng, 2, a, 7), k)
    check_topk(clustered_rows(rng, a), k)


@pytest.mark.parametrize("nq", [1, 2, 5, 16, 17, 40])
def test_topk_batch_sizes(nq):
    # around the switch between the two paths
    rng = np.random.default_rng(nq)
    s = (rng.standard_normal((nq, 32770)) * 20).astype(np.float32)
    s[:, 5] = 1e9  # a row-wide needle
    ids = check_topk(s, 512, "few-rows" if nq <= FEW_ROWS else "per-row")
    assert np.all(ids[:, 0] == 5)


def test_topk_no_active_blocks(gpu):
    ids = torch.full((4, 7), 99, dtype=torch.int32, device="cuda")
    st = gpu.qsa_block_topk(None, 4, 0, 7, ids.data_ptr(), None)
    assert st == 0
    torch.cuda.synchronize()
    assert np.all(ids.cpu().numpy() == -1)


@pytest.mark.parametrize("path", PATHS)
def test_topk_special_rows(path):
    a = 5000
    rows = [
        np.full(a, 1.5, np.float32),                         # all equal
        np.arange(a, dtype=np.float32),                      # increasing
        -np.arange(a, dtype=np.float32),                     # decreasing
        np.where(np.arange(a) % 2 == 0, -0.0, 0.0).astype(np.float32),  # signed zeros tie
        np.concatenate([np.full(10, np.inf), np.full(10, -np.inf),
                        np.zeros(a - 20)]).astype(np.float32),
        np.full(a, -np.inf, np.float32),
        np.full(a, np.finfo(np.float32).max, np.float32) * np.where(np.arange(a) % 3 == 0, -1, 1),
        np.full(a, np.float32(1e-45)) * (np.arange(a) % 4),  # subnormals
    ]
    s = np.ascontiguousarray(np.stack(rows).astype(np.float32))
    for k in (1, 7, 1000, 4096):
        ids = check_topk(s, k, path)[: s.shape[0]]
        assert topk_invariants(s, ids, k) == []
    ids = gpu_topk(s[3:4], 10)[0]
    assert ids.tolist() == list(range(10)), "-0.0 and +0.0 must tie (lower id first)"


def counting_rank_rows(rng, a):
    """Rows aimed at the one-workgroup top-k's counting rank (rank order of up
    to 1,024 pairs from 1,024 buckets of equal key ranges, a bucket capped at
    64 pairs, the sorting network past the cap): keys evenly spaced so that
    each bucket holds one, then one value repeated to fill its bucket exactly
    to the cap and one past it; a thousand consecutive floats (near-ties in
    one bucket) among random scores; and the widest key span, -Inf to +Inf."""
    even = (np.uint32(0x3F800000) + np.arange(a, dtype=np.uint32) * np.uint32(4096)).view(np.float32)
    rows = []
    for extra in (63, 64):  # the largest value's bucket: 64 pairs, then 65
        r = even.copy()
        r[rng.choice(a - 1, extra, replace=False)] = even[a - 1]
        rows.append(r)
    r = (rng.standard_normal(a) * 20).astype(np.float32)
    near = (np.float32(30.0).view(np.uint32) + np.arange(min(a, 1000), dtype=np.uint32)).view(np.float32)
    r[rng.choice(a, len(near), replace=False)] = near
    rows.append(r)
    r = rng.standard_normal(a).astype(np.float32)
    r[:4] = [np.inf, -np.inf, np.finfo(np.float32).max, -np.finfo(np.float32).max]
    rows.append(r)
    return np.ascontiguousarray(np.stack(rows).astype(np.float32))


@pytest.mark.parametrize("path", PATHS)
@pytest.mark.parametrize("a,k", [(1000, 1000), (1000, 300), (1024, 1024), (1025, 1025),
                                  (4097, 512), (32770, 512), (65538, 1024)])
def test_topk_counting_rank(a, k, path):
    s = counting_rank_rows(np.random.default_rng(a * 5 + k), a)
    ids = check_topk(s, k, path)
    assert topk_invariants(rows_for_path(s, path), ids, k) == []


def test_topk_deterministic():
    rng = np.random.default_rng(5)
    s = tie_rows(rng, 8, 40000, 50)
    assert np.array_equal(gpu_topk(s, 800), gpu_topk(s, 800))


# ------------------------------------------------------------ select ----

SELECT_CASES = [  # nq, heads, dim, active, k  (nq <= 8 with K <= 4096/nq fuse; the rest do not)
    (1, 4, 64, 512, 64), (1, 4, 128, 32770, 512), (1, 4, 128, 1000, 1000), (2, 4, 128, 5000, 100),
    (3, 2, 128, 777, 50), (8, 4, 128, 8193, 256), (1, 8, 256, 3000, 128), (1, 16, 256, 640, 64),
    (4, 4, 256, 2049, 300), (5, 2, 64, 65, 7), (1, 1, 4, 70, 5), (1, 4, 128, 63, 4096),
    (9, 4, 128, 3000, 256), (1, 4, 128, 131073, 64), (40, 4, 128, 2000, 100), (8, 8, 128, 300, 30),
    # decode at large k: more published words than 8 per thread, up to 128 rank workgroups
    (1, 4, 128, 32770, 4096), (4, 4, 128, 32770, 2048), (2, 4, 128, 33793, 3000),
    # a final group of 16, 1 and 17 blocks: the first two ride on the last full
    # group's workgroup of the 16-wave fused scorer, the third has its own
    (1, 4, 128, 1040, 64), (2, 4, 128, 32769, 512), (2, 4, 128, 1041, 64), (2, 4, 128, 80, 90),
]


@pytest.mark.parametrize("nq,heads,dim,active,k", SELECT_CASES)
def test_select_matches_separate_calls(nq, heads, dim, active, k):
    from sparse_attention_kv_qsa_amd import qsa_block_scores, qsa_block_select, qsa_block_topk
    q, kb = synth.make_random(nq, heads, dim, active, capacity=active + 3, seed=nq * 31 + active)
    qt, kt = torch.from_numpy(q).cuda(), torch.from_numpy(kb).cuda()
    s_sel, i_sel = qsa_block_select(qt, kt, k, active)
    s_sep = qsa_block_scores(qt, kt, active)
    i_sep = qsa_block_topk(s_sep, k)
    torch.cuda.synchronize()
    s_sel, i_sel, s_sep, i_sep = (x.cpu().numpy() for x in (s_sel, i_sel, s_sep, i_sep))
    assert np.array_equal(s_sel, s_sep), "select's scores differ from qsa_block_scores"
    assert np.array_equal(i_sel, i_sep), "select's ids differ from qsa_block_topk"
    check_scores(s_sel, ORC.scores_f64(q, kb, active))
    assert np.array_equal(i_sel, ORC.topk(s_sel, k))


@pytest.mark.parametrize("nq,active", [(1, 32770), (2, 1040), (1, 65)])
def test_select_winners_in_merged_tail(nq, active):
    """The best blocks sit in the final, partial group, whose scores and group
    words the fused scorer's last workgroup produces besides its own group."""
    from sparse_attention_kv_qsa_amd import qsa_block_select
    q, kb = synth.make_random(nq, 4, 128, active, capacity=active + 2, seed=active + nq)
    tail = np.arange(64 * ((active - 1) // 64), active)
    kb[tail] = 3.0 * q[np.arange(len(tail)) % nq]  # these blocks score highest for their query
    qt, kt = torch.from_numpy(q).cuda(), torch.from_numpy(kb).cuda()
    k = 24
    s, ids = qsa_block_select(qt, kt, k, active)
    torch.cuda.synchronize()
    s, ids = s.cpu().numpy(), ids.cpu().numpy()
    check_scores(s, ORC.scores_f64(q, kb, active))
    assert np.array_equal(ids, ORC.topk(s, k))
    for n in range(nq):
        assert set(tail[np.arange(len(tail)) % nq == n].tolist()) <= set(ids[n].tolist())


def test_select_edges(gpu):
    from sparse_attention_kv_qsa_amd import qsa_block_select
    q, kb = synth.make_random(2, 4, 128, 300, capacity=303, seed=9)
    qt, kt = torch.from_numpy(q).cuda(), torch.from_numpy(kb).cuda()
    # k = 0: scores only, ids untouched
    ids = torch.full((2, 0), 7, dtype=torch.int32, device="cuda")
    s, _ = qsa_block_select(qt, kt, 0, 300, ids=ids)
    torch.cuda.synchronize()
    check_scores(s.cpu().numpy(), ORC.scores_f64(q, kb, 300))
    # no active blocks: all -1
    ids = torch.full((2, 5), 7, dtype=torch.int32, device="cuda")
    _, ids = qsa_block_select(qt, kt, 5, 0, ids=ids)
    torch.cuda.synchronize()
    assert np.all(ids.cpu().numpy() == -1)
    # mass ties through the fused path: every summary identical
    kb_same = np.ascontiguousarray(np.broadcast_to(kb[:1], (5000, 4, 128)))
    s, ids = qsa_block_select(qt, torch.from_numpy(kb_same).cuda(), 100, 5000)
    torch.cuda.synchronize()
    s = s.cpu().numpy()
    assert np.all(s == s[:, :1])
    assert np.array_equal(ids.cpu().numpy(), np.tile(np.arange(100, dtype=np.int32), (2, 1)))


# ------------------------------------------------- full workloads ----

def oracle_scores_rows(q, kblk, active):
    """FP64 oracle scores of every query row, rows spread over host threads
    (the C oracle releases the GIL)."""
    import concurrent.futures as cf
    threads = max(1, min(16, len(os.sched_getaffinity(0)), q.shape[0]))
    chunks = [r for r in np.array_split(np.arange(q.shape[0]), threads) if len(r)]
    with cf.ThreadPoolExecutor(threads) as ex:
        parts = list(ex.map(lambda r: ORC.scores_f64(q[r], kblk, active), chunks))
    return np.concatenate(parts, axis=0)


def margins(s, s64, ids, k):
    """Score error against the gate, over the call and per row, and how the
    selection on the GPU's scores compares with the selection on the FP64
    ones (a diagnostic, never a gate: near-ties legitimately flip)."""
    err = np.abs(s.astype(np.float64) - s64)
    row_scale = np.abs(s64).max(axis=1)
    row_ratio = err.max(axis=1) / (SCORE_TOL * np.where(row_scale > 0, row_scale, 1.0))
    ids64 = ORC.topk_f64(np.ascontiguousarray(s64), k)
    same_rows = np.all(ids == ids64, axis=1)
    m = min(k, s.shape[1])
    set_diff = [len(set(a[:m].tolist()) ^ set(b[:m].tolist())) // 2 for a, b in zip(ids, ids64)]
    return {
        "gate_ratio": float(err.max() / (SCORE_TOL * np.abs(s64).max())),
        "worst_row_ratio": float(row_ratio.max()),
        "worst_row": int(row_ratio.argmax()),
        "fp64_same_selection_rows": int(same_rows.sum()),
        "rows": int(s.shape[0]),
        "fp64_selected_cells_differ": int(sum(set_diff)),
        "selected_cells": int(s.shape[0] * m),
        "fp64_rank_slots_differ": int(np.sum(ids != ids64)),
    }


@pytest.mark.slow
@pytest.mark.parametrize("mode", ["auto", "fp32", "bf16x3", "select"])
@pytest.mark.parametrize("name", list(synth.WORKLOADS))
def test_workload_parity(name, mode):
    w = synth.WORKLOADS[name]
    print(f"\n[workload {name} {mode}] nq={w.nq} A={w.active} C={w.capacity} K={w.K} k={w.k}",
          flush=True)
    bt = synth.make_batch(w)
    from sparse_attention_kv_qsa_amd import qsa_block_scores_ex, qsa_block_select, qsa_block_topk
    qt, kt = torch.from_numpy(bt.q).cuda(), torch.from_numpy(bt.kblk).cuda()
    if mode == "select":
        s_t, ids_t = qsa_block_select(qt, kt, w.k, w.active)
        s_t2, ids_t2 = qsa_block_select(qt, kt, w.k, w.active)
    else:
        s_t = qsa_block_scores_ex(qt, kt, w.active, mode=mode)
        ids_t = qsa_block_topk(s_t, w.k)
        s_t2 = qsa_block_scores_ex(qt, kt, w.active, mode=mode)
        ids_t2 = qsa_block_topk(s_t2, w.k)
    torch.cuda.synchronize()
    s, ids = s_t.cpu().numpy(), ids_t.cpu().numpy()
    assert np.array_equal(s, s_t2.cpu().numpy()) and np.array_equal(ids, ids_t2.cpu().numpy())
    assert np.all(np.isfinite(s)), "poisoned capacity rows were read"

    # FP64 scores of every row: the gate over the whole call.
    s64 = oracle_scores_rows(bt.q, bt.kblk, w.active)
    ratio = check_scores(s, s64)
    want = ORC.topk(s, w.k)
    assert np.array_equal(ids, want), f"{np.sum(np.any(ids != want, axis=1))} rows differ"

    rep = {"workload": name, "mode": mode, **margins(s, s64, ids, w.k)}
    assert rep["gate_ratio"] == pytest.approx(ratio)
    print(f"[workload {name} {mode}] margins {rep}", flush=True)
    out_dir = os.environ.get("QSA_MARGINS_DIR")
    if out_dir:
        import json
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, f"{name}_{mode}.json"), "w") as f:
            json.dump(rep, f)

    if w.tie_vectors:
        # blocks built from the same vector score bitwise-equal within a row
        plain = np.ones(w.active, bool)
        plain[bt.needle_blocks] = False
        for c in range(3):
            cols = s[:, plain & (bt.tie_assign == c)]
            assert np.all(cols == cols[:, :1])
    if len(bt.needle_blocks):
        # a needle built from query j sits far above j's other scores
        sel = set()
        for b, j in zip(bt.needle_blocks[:50], bt.needle_queries[:50]):
            sel.add(int(b) in set(ids[j].tolist()))
        assert sel == {True}


# ------------------------------------------------ sharding, on one GPU ----

@pytest.mark.parametrize("nq,active,k,ties", [(256, 32770, 512, 0), (1, 32770, 512, 0),
                                               (64, 20000, 300, 7), (3, 5000, 1024, 0)])
def test_sharded_select_merges_exactly(nq, active, k, ties):
    """The block-range sharding of the selection: G = 8 shards each select
    their own top k over their block range (ids local to the shard); the
    shards' winners, concatenated in shard order, are selected again.  A
    block's score does not depend on which call or tile holds it, and equal
    scores resolve by concatenation index, which is the global id order
    (shards in range order, each list in rank order), so the merged selection
    equals the one-call selection id for id."""
    from sparse_attention_kv_qsa_amd import qsa_block_select, qsa_block_topk
    G = 8
    rng = np.random.default_rng(active + nq)
    q = rng.standard_normal((nq, 4, 128)).astype(np.float32)
    if ties:
        vec = rng.standard_normal((ties, 4, 128)).astype(np.float32)
        kb = np.ascontiguousarray(vec[rng.integers(0, ties, active)])
    else:
        kb = rng.standard_normal((active, 4, 128)).astype(np.float32)
    qt, kt = torch.from_numpy(q).cuda(), torch.from_numpy(kb).cuda()
    s_all, ids_all = qsa_block_select(qt, kt, k, active)
    bounds = [active * g // G for g in range(G + 1)]
    cand_s, cand_id, shard_s = [], [], []
    for g in range(G):
        lo, hi = bounds[g], bounds[g + 1]
        s_g, ids_g = qsa_block_select(qt, kt[lo:hi].contiguous(), k, hi - lo)
        shard_s.append(s_g)
        ok = ids_g >= 0
        sel = torch.gather(s_g, 1, ids_g.clamp(min=0).long())
        # padding slots (k > shard size) take -inf and an id past every block
        cand_s.append(torch.where(ok, sel, torch.full_like(sel, -float("inf"))))
        cand_id.append(torch.where(ok, ids_g + lo, torch.full_like(ids_g, 2 ** 30)))
    cs = torch.cat(cand_s, dim=1).contiguous()
    ci = torch.cat(cand_id, dim=1)
    pick = qsa_block_topk(cs, k)
    merged = torch.gather(ci, 1, pick.clamp(min=0).long())
    merged = torch.where(pick >= 0, merged, torch.full_like(merged, -1))
    torch.cuda.synchronize()
    assert torch.equal(merged.int(), ids_all)
    # and the shards' scores are the one call's scores, bit for bit
    assert torch.equal(torch.cat(shard_s, dim=1), s_all)
