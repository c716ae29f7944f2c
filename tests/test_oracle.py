"""Pins of the CPU oracle against things other than itself (no GPU needed).

The pages print no worked example, score values or id lists, so the oracle is
pinned by: a hand-worked example (tests/golden/hand_3block.txt), exact integer
inputs vs numpy int64 matmul, exact rationals, numpy float64 matmul, the
brute-force rank definition, numpy lexsort, closed-form special rows and
invariants.  ``test_mutants_are_caught`` plants plausible mistakes in copies of
the oracle's C source and shows that every one fails some pin.
"""
from __future__ import annotations

import math
import os
import random
import re
import tempfile
from fractions import Fraction

import numpy as np
import pytest

import oracle
from checks import brute_force_topk, score_gate, topk_invariants

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_3block.txt")
ORC = oracle.default()


def load_hand_example():
    heads = dim = None
    q, b, scores, topks = [], [], {}, []
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, rest = line.split(None, 1)
            if key == "heads":
                heads = int(rest)
            elif key == "dim":
                dim = int(rest)
            elif key == "q":
                q.append([float(x) for x in rest.split()])
            elif key == "b":
                b.append([float(x) for x in rest.split()])
            elif key == "scores":
                i, vals = rest.split(":")
                scores[int(i)] = [float(x) for x in vals.split()]
            elif key == "topk":
                head, vals = rest.split(":")
                i, k = (int(x) for x in head.split())
                topks.append((i, k, [int(x) for x in vals.split()]))
    q = np.array(q, np.float32).reshape(-1, heads, dim)
    b = np.array(b, np.float32).reshape(-1, heads, dim)
    return q, b, scores, topks


# ----------------------------------------------------------------- pins ----

def pin_hand_example(orc):
    q, b, scores, topks = load_hand_example()
    s = orc.scores_f64(q, b, b.shape[0])
    for i, want in scores.items():
        if list(s[i]) != want:
            return f"hand scores row {i}: {list(s[i])} != {want}"
    s32 = s.astype(np.float32)
    for i, k, want in topks:
        got = orc.topk(s32[i:i + 1], k)[0].tolist()
        if got != want:
            return f"hand top-k q{i} k={k}: {got} != {want}"
    return None


INT_SHAPES = [(1, 1, 1, 1), (2, 3, 5, 7), (5, 2, 7, 3), (3, 4, 64, 33), (7, 1, 12, 19), (4, 4, 128, 9)]


def pin_integer_exact(orc):
    """Small-integer inputs: every fp64 partial sum is an exact integer, so the
    oracle must equal numpy's int64 matmul exactly (an independent routine)."""
    rng = np.random.default_rng(1)
    for nq, heads, dim, a in INT_SHAPES:
        q = rng.integers(-8, 9, (nq, heads, dim))
        kb = rng.integers(-8, 9, (a + 2, heads, dim))
        want = q.reshape(nq, -1).astype(np.int64) @ kb[:a].reshape(a, -1).astype(np.int64).T
        got = orc.scores_f64(q.astype(np.float32), kb.astype(np.float32), a)
        if not np.array_equal(got, want.astype(np.float64)):
            return f"integer shape {(nq, heads, dim, a)}: mismatch"
    return None


def pin_float64_matmul(orc):
    rng = np.random.default_rng(2)
    for nq, heads, dim, a in [(3, 4, 64, 50), (2, 3, 5, 17), (6, 1, 300, 11)]:
        q = rng.standard_normal((nq, heads, dim)).astype(np.float32)
        kb = rng.standard_normal((a, heads, dim)).astype(np.float32)
        want = q.reshape(nq, -1).astype(np.float64) @ kb.reshape(a, -1).astype(np.float64).T
        got = orc.scores_f64(q, kb, a)
        scale = np.abs(want).max()
        if np.abs(got - want).max() > 1e-12 * scale:
            return f"float64 matmul shape {(nq, heads, dim, a)}: mismatch"
    return None


def pin_exact_rationals(orc):
    """Exact value by fractions.Fraction; the FP64 sum may differ only by the
    rounding of its K-1 additions: |s64 - exact| <= (K-1) * 2^-53 * sum|products|."""
    rng = np.random.default_rng(3)
    nq, heads, dim, a = 2, 2, 3, 4
    q = rng.standard_normal((nq, heads, dim)).astype(np.float32)
    kb = rng.standard_normal((a, heads, dim)).astype(np.float32)
    got = orc.scores_f64(q, kb, a)
    K = heads * dim
    for i in range(nq):
        for b in range(a):
            prods = [Fraction(float(x)) * Fraction(float(y))
                     for x, y in zip(q[i].ravel(), kb[b].ravel())]
            exact = sum(prods, Fraction(0))
            bound = (K - 1) * 2.0 ** -53 * float(sum(abs(p) for p in prods))
            if abs(Fraction(got[i, b]) - exact) > Fraction(bound):
                return f"rational ({i},{b}) outside the rounding bound"
    return None


TIE_VALUES = [-1.0, -0.0, 0.0, 1.0, 2.0]


def pin_topk_brute_force(orc):
    rnd = random.Random(4)
    for a in range(0, 13):
        for _ in range(6):
            row = [rnd.choice(TIE_VALUES) for _ in range(a)]
            for k in range(0, a + 3):
                got = orc.topk(np.array([row], np.float32).reshape(1, a), k)[0].tolist()
                if got != brute_force_topk(row, k):
                    return f"brute force row={row} k={k}: {got}"
    return None


def pin_topk_lexsort(orc):
    rng = np.random.default_rng(5)
    for a, k in [(100, 10), (1000, 64), (4097, 512), (300, 300), (50, 80)]:
        s = np.round(rng.standard_normal((4, a)) * 4).astype(np.float32)  # many ties
        got = orc.topk(s, k)
        for i in range(4):
            order = np.lexsort((np.arange(a), -s[i].astype(np.float64)))[: min(k, a)]
            want = np.full(k, -1, np.int64)
            want[: len(order)] = order
            if not np.array_equal(got[i], want):
                return f"lexsort a={a} k={k} row {i}"
    return None


def pin_topk_f64_lexsort(orc):
    """The FP64 selection (a diagnostic: how often the fp32 scores select what
    the FP64 ones do) against numpy lexsort on float64 rows whose values differ
    only below fp32 precision: neighbours one FP64 ulp apart, values split by
    2^-40 relative, exact ties, signed zeros and infinities.  A NaN must be
    reported."""
    rng = np.random.default_rng(12)
    for a, k in [(64, 10), (500, 77), (2000, 300), (37, 50)]:
        base = np.round(rng.standard_normal(a) * 3)
        jitter = rng.integers(-2, 3, a).astype(np.float64)
        rows = [
            base + jitter * 2.0 ** -40 * np.maximum(np.abs(base), 1.0),      # below fp32's ulp
            np.where(rng.random(a) < 0.5, base, np.nextafter(base, np.inf)),  # one FP64 ulp apart
            np.where(rng.random(a) < 0.3, -0.0, np.where(rng.random(a) < 0.5, 0.0, base)),
            np.where(rng.random(a) < 0.05, np.inf, np.where(rng.random(a) < 0.05, -np.inf, base)),
        ]
        s = np.ascontiguousarray(np.stack(rows))
        got = orc.topk_f64(s, k)
        for i in range(len(rows)):
            order = np.lexsort((np.arange(a), -s[i]))[: min(k, a)]
            want = np.full(k, -1, np.int64)
            want[: len(order)] = order
            if not np.array_equal(got[i], want):
                return f"FP64 lexsort a={a} k={k} row {i}"
    # narrowing to fp32 would merge the first row's neighbours into ties
    near = np.array([[1.0, 1.0 + 2.0 ** -40, 1.0 + 2.0 ** -41]])
    if orc.topk_f64(near, 3)[0].tolist() != [1, 2, 0]:
        return "FP64 selection lost differences below fp32 precision"
    bad = np.array([[0.5, np.nan, 1.0]])
    try:
        orc.topk_f64(bad, 2)
    except oracle.OracleError:
        return None
    return "a NaN FP64 score was not reported"


def pin_topk_special_rows(orc):
    a, k = 37, 9
    const = np.full((1, a), 3.5, np.float32)
    dec = np.arange(a, 0, -1, dtype=np.float32)[None]
    inc = np.arange(a, dtype=np.float32)[None]
    checks = [
        (const, list(range(k))),
        (dec, list(range(k))),
        (inc, list(range(a - 1, a - 1 - k, -1))),
    ]
    for s, want in checks:
        if orc.topk(s, k)[0].tolist() != want:
            return "special row"
    full = orc.topk(inc, a)[0].tolist()
    if full != list(range(a - 1, -1, -1)):
        return "k = A is not the full sorted permutation"
    if orc.topk(np.zeros((2, 0), np.float32), 3).tolist() != [[-1, -1, -1]] * 2:
        return "A = 0 must give all -1"
    return None


def pin_topk_invariants(orc):
    rng = np.random.default_rng(6)
    for a, k in [(200, 17), (513, 64), (64, 64), (10, 30)]:
        s = np.round(rng.standard_normal((3, a)) * 3).astype(np.float32)
        bad = topk_invariants(s, orc.topk(s, k), k)
        if bad:
            return f"invariants a={a} k={k}: {bad[:2]}"
    return None


def pin_active_rows_only(orc):
    """Rows past active_blocks are never read: NaN there changes nothing."""
    q, kb = np.ones((2, 2, 3), np.float32), np.ones((6, 2, 3), np.float32)
    kb[4:] = np.nan
    s = orc.scores_f64(q, kb, 4)
    if not np.all(s == 6.0):
        return "poison rows were read"
    return None


# ------------------------------------------ decode attention pins ----
# (page "#3102 perf(hip): enable wave32 QSA decode attention and MMVQ row reuse
# on gfx12", Summary item 1: attention of each query over the cells of its
# selected blocks; the formula is scaled dot-product attention per head)

POISON = 1e30  # finite, so a mutant that reads masked cells changes the result without NaN


def attn_case(rng, nq, heads, dim, n_cells, extra=8):
    q = rng.standard_normal((nq, heads, dim)).astype(np.float32)
    kc = rng.standard_normal((n_cells + extra, heads, dim)).astype(np.float32)
    vc = rng.standard_normal((n_cells + extra, heads, dim)).astype(np.float32)
    kc[n_cells:] = POISON
    vc[n_cells:] = POISON
    return q, kc, vc


def numpy_attn(q, kc, vc, ids, n_cells, scale):
    """Vectorised FP64 attention written independently of the oracle's loops."""
    nq, heads, dim = q.shape
    out = np.zeros((nq, heads, dim))
    for i in range(nq):
        cells = np.array([4 * b + e for b in ids[i] if b >= 0 for e in range(4)
                          if 4 * b + e < n_cells], dtype=np.int64)
        if cells.size == 0:
            continue
        kk = kc[cells].astype(np.float64)            # [n][heads][dim]
        vv = vc[cells].astype(np.float64)
        s = scale * np.einsum("hd,nhd->hn", q[i].astype(np.float64), kk)
        w = np.exp(s - s.max(axis=1, keepdims=True))
        out[i] = np.einsum("hn,nhd->hd", w, vv) / w.sum(axis=1)[:, None]
    return out


def pin_attn_single_cell(orc):
    """One attended cell: its value row, exactly."""
    rng = np.random.default_rng(21)
    q, kc, vc = attn_case(rng, 1, 2, 8, n_cells=9)
    out = orc.sparse_decode_attn_f64(q, kc, vc, np.array([[2, -1]], np.int32), 9, 0.3)
    if not np.array_equal(out[0], vc[8].astype(np.float64)):
        return "single attended cell does not return its value row"
    return None


def pin_attn_uniform_weights(orc):
    """q = 0: every weight is 1, the output is the exact mean of the attended rows."""
    rng = np.random.default_rng(22)
    q, kc, vc = attn_case(rng, 1, 2, 4, n_cells=10)
    q[:] = 0
    ids = np.array([[0, 2]], np.int32)  # cells 0-3 and 8, 9 (10, 11 masked)
    out = orc.sparse_decode_attn_f64(q, kc, vc, ids, 10, 1.0)
    cells = [0, 1, 2, 3, 8, 9]
    for h in range(2):
        for d in range(4):
            exact = sum(Fraction(float(vc[c, h, d])) for c in cells) / len(cells)
            if abs(Fraction(out[0, h, d]) - exact) > Fraction(1, 2**50) * max(1, abs(exact)):
                return f"uniform weights: head {h} dim {d} is not the mean"
    return None


def pin_attn_numpy(orc):
    """Random tiny cases (padding, a repeated block, a partial last block) vs numpy."""
    rng = np.random.default_rng(23)
    for nq, heads, dim, n_cells, ids in [
            (2, 3, 8, 22, [[5, -1, 0, 3], [1, 1, -1, 4]]),
            (1, 1, 4, 7, [[1, 0, -1, -1]]),
            (3, 2, 16, 40, [[9, 2, 7, 0], [-1, -1, -1, -1], [3, 8, 6, 1]])]:
        q, kc, vc = attn_case(rng, nq, heads, dim, n_cells)
        ids = np.array(ids, np.int32)
        got = orc.sparse_decode_attn_f64(q, kc, vc, ids, n_cells, 0.25)
        want = numpy_attn(q, kc, vc, ids, n_cells, 0.25)
        if not np.allclose(got, want, rtol=1e-12, atol=1e-12):
            return f"differs from numpy at nq={nq} heads={heads} dim={dim}"
    return None


def pin_attn_two_cells_closed_form(orc):
    """Two cells with scores 1000 and 998: weights 1/(1+e^-2) and e^-2/(1+e^-2)."""
    q = np.zeros((1, 1, 4), np.float32)
    q[0, 0, 0] = 1.0
    kc = np.zeros((8, 1, 4), np.float32)
    kc[0, 0, 0], kc[1, 0, 0] = 1000.0, 998.0
    vc = np.zeros((8, 1, 4), np.float32)
    vc[0, 0] = [1, 2, 3, 4]
    vc[1, 0] = [-4, 0, 0.5, 8]
    kc[2:] = POISON
    vc[2:] = POISON
    out = orc.sparse_decode_attn_f64(q, kc, vc, np.array([[0]], np.int32), 2, 1.0)
    e = math.exp(-2.0)
    want = (vc[0, 0].astype(np.float64) + e * vc[1, 0].astype(np.float64)) / (1 + e)
    if not np.allclose(out[0, 0], want, rtol=1e-15, atol=1e-15):
        return "two-cell closed form"
    return None


def pin_attn_invariants(orc):
    """List order does not matter; padding and power-of-two value scaling are exact."""
    rng = np.random.default_rng(24)
    q, kc, vc = attn_case(rng, 2, 2, 8, n_cells=30)
    ids = np.array([[6, 0, 3, 5], [2, 7, 1, 4]], np.int32)
    base = orc.sparse_decode_attn_f64(q, kc, vc, ids, 30, 0.5)
    if not np.allclose(orc.sparse_decode_attn_f64(q, kc, vc, ids[:, ::-1].copy(), 30, 0.5), base,
                       rtol=1e-13, atol=1e-13):
        return "block order changes the result"
    padded = np.array([[6, -1, 0, 3, -1, 5], [-1, 2, 7, 1, 4, -1]], np.int32)
    if not np.array_equal(orc.sparse_decode_attn_f64(q, kc, vc, padded, 30, 0.5), base):
        return "padding changes the result"
    if not np.array_equal(orc.sparse_decode_attn_f64(q, kc, vc * 2, ids, 30, 0.5), base * 2):
        return "value scaling is not exact"
    empty = orc.sparse_decode_attn_f64(q, kc, vc, np.full((2, 3), -1, np.int32), 30, 0.5)
    if not np.all(empty == 0):
        return "no attended cell must give zeros"
    return None


# ---------------------------------------------------- int8 pool ----
# (an int8 key/value pool: one code per (cell, head, d), one binary16 scale
# per (cell, head); page "#3224 [Engine] perf(hip): tune RDNA4 QSA prompt WMMA
# path (STRATA_HIP_WMMA stays opt-in)", Summary item 2, and the int8 rows of
# the decode-attention table of "#3102 perf(hip): ...")

def pin_half_decoding(orc):
    """The oracle's binary16 decoding agrees with numpy's float16 on all 65,536
    bit patterns (sign, zeros, subnormals, infinities and NaN included)."""
    b = np.arange(65536, dtype=np.uint16)
    ref = b.view(np.float16).astype(np.float64)
    got = orc.half_to_f64(b)
    nan = np.isnan(ref)
    if not np.array_equal(np.isnan(got), nan):
        return "half decoding: NaN patterns differ"
    if not np.array_equal(got[~nan], ref[~nan]) or \
            not np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan])):
        return "half decoding differs from numpy float16"
    return None


def i8_case(rng, nq, heads, dim, n_cells, extra=8):
    q = rng.standard_normal((nq, heads, dim)).astype(np.float32)
    pools = []
    for _ in range(2):
        codes = rng.integers(-127, 128, (n_cells + extra, heads, dim)).astype(np.int8)
        scales = rng.uniform(0.005, 0.05, (n_cells + extra, heads)).astype(np.float16)
        scales[n_cells:] = np.float16(60000.0)  # masked cells: a huge but finite scale
        pools += [codes, scales.view(np.uint16)]
    return q, pools


def dequantize(codes, scale_bits):
    """code * scale, exact in float32 (an 8-bit code times an 11-bit significand)."""
    return codes.astype(np.float32) * scale_bits.view(np.float16).astype(np.float32)[..., None]


def pin_attn_i8_dequantized(orc):
    """The int8 pool gives the attention of its dequantised fp32 rows: the same
    FP64 values as the fp32 attention on them, and numpy's within 1e-12."""
    rng = np.random.default_rng(31)
    for nq, heads, dim, n_cells, ids in [
            (2, 3, 8, 22, [[5, -1, 0, 3], [1, 1, -1, 4]]),
            (3, 2, 16, 40, [[9, 2, 7, 0], [-1, -1, -1, -1], [3, 8, 6, 1]])]:
        q, (kq, ks, vq, vs) = i8_case(rng, nq, heads, dim, n_cells)
        ids = np.array(ids, np.int32)
        got = orc.sparse_decode_attn_i8_f64(q, kq, ks, vq, vs, ids, n_cells, 0.25)
        kc, vc = dequantize(kq, ks), dequantize(vq, vs)
        if not np.array_equal(got, orc.sparse_decode_attn_f64(q, kc, vc, ids, n_cells, 0.25)):
            return f"int8 pool differs from fp32 attention on its dequantised rows (dim={dim})"
        if not np.allclose(got, numpy_attn(q, kc, vc, ids, n_cells, 0.25), rtol=1e-12, atol=1e-12):
            return f"int8 pool differs from numpy on its dequantised rows (dim={dim})"
    return None


def pin_attn_i8_single_cell(orc):
    """One attended cell: code * scale of its value row, exactly, signs included."""
    rng = np.random.default_rng(32)
    q, (kq, ks, vq, vs) = i8_case(rng, 1, 2, 8, n_cells=9)
    vq[8, 1, :4] = [-128, 127, -1, 0]
    out = orc.sparse_decode_attn_i8_f64(q, kq, ks, vq, vs, np.array([[2, -1]], np.int32), 9, 0.3)
    want = vq[8].astype(np.float64) * vs[8].view(np.float16).astype(np.float64)[:, None]
    if not np.array_equal(out[0], want):
        return "int8 single cell is not code * scale"
    return None


PINS = [pin_hand_example, pin_integer_exact, pin_float64_matmul, pin_exact_rationals,
        pin_topk_brute_force, pin_topk_lexsort, pin_topk_f64_lexsort, pin_topk_special_rows,
        pin_topk_invariants, pin_active_rows_only, pin_attn_single_cell,
        pin_attn_uniform_weights, pin_attn_numpy, pin_attn_two_cells_closed_form,
        pin_attn_invariants, pin_half_decoding, pin_attn_i8_dequantized,
        pin_attn_i8_single_cell]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pins(pin):
    assert pin(ORC) is None


# -------------------------------------------------- further properties ----

def test_power_of_two_scaling_is_exact():
    rng = np.random.default_rng(7)
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    kb = rng.standard_normal((20, 4, 16)).astype(np.float32)
    s = ORC.scores_f64(q, kb, 20)
    assert np.array_equal(ORC.scores_f64(q * 4, kb, 20), s * 4)
    assert np.array_equal(ORC.scores_f64(q, kb * 0.5, 20), s * 0.5)


def test_block_permutation_permutes_scores_bitwise():
    rng = np.random.default_rng(8)
    q = rng.standard_normal((3, 4, 16)).astype(np.float32)
    kb = rng.standard_normal((30, 4, 16)).astype(np.float32)
    perm = rng.permutation(30)
    assert np.array_equal(ORC.scores_f64(q, kb[perm], 30), ORC.scores_f64(q, kb, 30)[:, perm])


def test_nan_score_is_reported():
    s = np.zeros((1, 5), np.float32)
    s[0, 3] = np.nan
    with pytest.raises(oracle.OracleError):
        ORC.topk(s, 2)


def test_infinities_order_naturally():
    s = np.array([[1.0, np.inf, -np.inf, 0.0]], np.float32)
    assert ORC.topk(s, 4)[0].tolist() == [1, 0, 3, 2]


def test_f64_selection_matches_fp32_on_exact_values():
    # consistency only (both share the sort); pin_topk_f64_lexsort is the pin
    rng = np.random.default_rng(9)
    s = np.round(rng.standard_normal((4, 300)) * 8)
    assert np.array_equal(ORC.topk_f64(s, 40), ORC.topk(s.astype(np.float32), 40))


# ------------------------------------------------ negative controls ----

def test_checkers_catch_planted_result_errors():
    rng = np.random.default_rng(10)
    s = np.round(rng.standard_normal((1, 400)) * 3).astype(np.float32)
    k = 50
    ids = ORC.topk(s, k)
    assert topk_invariants(s, ids, k) == []
    # swap two tied ids inside the selection
    row = ids[0].copy()
    v = s[0, row]
    r = next(r for r in range(k - 1) if v[r] == v[r + 1])
    bad = ids.copy()
    bad[0, r], bad[0, r + 1] = row[r + 1], row[r]
    assert topk_invariants(s, bad, k)
    # nudge the last selected score one ulp below the best unselected one
    s2 = s.copy()
    last = ids[0, -1]
    mask = np.ones(400, bool)
    mask[ids[0]] = False
    best_unsel = s[0, mask].max()
    s2[0, last] = np.nextafter(best_unsel, np.float32(-np.inf))
    assert topk_invariants(s2, ids, k) or not np.array_equal(ORC.topk(s2, k), ids)


def test_score_gate_catches_a_shift():
    rng = np.random.default_rng(11)
    s64 = rng.standard_normal((4, 100)) * 20
    ok, _ = score_gate(s64.astype(np.float32), s64)
    assert ok
    bad = s64.astype(np.float32).astype(np.float64)
    bad[2, 7] += 2e-6 * np.abs(s64).max()
    assert not score_gate(bad, s64)[0]


# Each mutant is a plausible mistake in the oracle's C source: (pattern, replacement).
MUTANTS = {
    "dropped last head": (r"h < heads; \+\+h", "h < heads - 1; ++h"),
    "dropped first dim term": (r"int64_t d = 0; d < dim", "int64_t d = 1; d < dim"),
    "wrong sign": (r"s \+= qv \* kv;", "s -= qv * kv;"),
    "q squared": (r"s \+= qv \* kv;", "s += qv * qv;"),
    "kblk transposed": (r"kblk\[\(b \* heads \+ h\) \* dim \+ d\]", "kblk[(b * dim + d) * heads + h]"),
    "q index drops the head": (r"q\[\(i \* heads \+ h\) \* dim \+ d\]", "q[i * heads * dim + d]"),
    "output transposed": (r"out\[i \* active_blocks \+ b\]", "out[b * nq + i]"),
    "ties to the higher id": (r"if \(a->id < b->id\) return -1;\n  if \(a->id > b->id\) return 1;",
                              "if (a->id > b->id) return -1;\n  if (a->id < b->id) return 1;"),
    "ascending order": (r"if \(a->score > b->score\) return -1;\n  if \(a->score < b->score\) return 1;",
                        "if (a->score < b->score) return -1;\n  if (a->score > b->score) return 1;"),
    "pad with zero": (r": -1;", ": 0;"),
    "FP64 selection narrowed to float": (r"c\[b\]\.score = s;", "c[b].score = (float)s;"),
    "FP64 selection misses a NaN": (r"(const double s = scores\[i \* active_blocks \+ b\];\n\s*)if \(isnan\(s\)\)",
                                    r"\1if (0)"),
    "signed-zero unequal": (r"c\[b\]\.score = \(double\)s;", "c[b].score = signbit(s) ? -1e-300 : (double)s;"),
    "score via float accumulation": (r"double s = 0\.0;", "float s = 0.0f;"),
    "attention without the scale": (r"s\[c\] = scale \* dot;", "s[c] = dot;"),
    "attention reads masked cells": (r"if \(4 \* b \+ e < n_cells\)", "if (4 * b + e <= n_cells)"),
    "attention divides by the count": (r"o\[d\] /= l;", "o[d] /= (double)n;"),
    "attention values from the keys": (r"\+= w \* \(double\)vc\[", "+= w * (double)kc["),
    "attention three cells per block": (r"e < 4; \+\+e", "e < 3; ++e"),
    "attention without the max shift": (r"exp\(s\[c\] - m\)", "exp(s[c])"),
    "attention keeps stale output": (r"o\[d\] = 0\.0;", "(void)o;"),
    "int8 key scale from the value scales": (r"oracle_half_to_double\(kscale\[r\]\)",
                                             "oracle_half_to_double(vscale[r])"),
    "int8 codes read unsigned": (r"\(double\)kcode\[r \* dim \+ d\]",
                                 "(double)(uint8_t)kcode[r * dim + d]"),
    "int8 scale per cell, not per head": (r"kscale\[r\]", "kscale[cell[c]]"),
    "int8 values without their scale": (r"\(\(double\)vcode\[r \* dim \+ d\] \* vs\)",
                                        "((double)vcode[r * dim + d])"),
    "half exponent bias off by one": (r"e - 25", "e - 24"),
    "half subnormals flushed": (r"v = ldexp\(\(double\)f, -24\);", "v = 0.0;"),
    "half sign dropped": (r"return sign \? -v : v;", "return v;"),
    "half implicit bit dropped": (r"1024 \+ f", "f"),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutants_are_caught(name):
    pattern, repl = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "qsa_oracle.c")).read()
    mutated, n = re.subn(pattern, repl, src)
    assert n >= 1, f"mutation {name!r} did not apply"
    with tempfile.TemporaryDirectory() as d:
        path = os.path.join(d, "mutant.c")
        with open(path, "w") as f:
            f.write(mutated)
        lib = oracle.compile_source(path, os.path.join(d, "libmutant.so"))
        mutant = oracle.load_from(lib)
        failures = [p.__name__ for p in PINS if p(mutant) is not None]
    assert failures, f"no pin catches the mutant {name!r}"
