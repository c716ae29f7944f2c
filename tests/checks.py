"""Checkers shared by the oracle pins and the GPU parity tests.

These do not compute selections themselves beyond tiny brute force; they
judge a result against what the definition fixes:

* ``score_gate``: max |s - s64| <= tol * max |s64| over the whole call (the
  FP64-relative gate; tol = 1e-6).
* ``brute_force_topk``: rank(b) = #{c : s[c] > s[b] or (s[c] == s[b] and c < b)},
  the definition of the selection order written out, for tiny rows only.
* ``topk_invariants``: properties any correct selection has (distinct ids in
  range, rank order, selected >= unselected, threshold ties taken lowest-id
  first, -1 padding past the row length).
* ``attn_limit``: the decode-attention gate for each (query, head).
"""
from __future__ import annotations

import numpy as np

# Decode attention gate, per query i and head h:
#   max_d |out - out64| <= max_{c} |v[c][h]| * (ATTN_TOL + ATTN_SCORE_TOL * scale * max_c sum_d |q_d k_cd|)
# over the attended cells c.  The output is a convex combination of value
# rows.  An fp32 score s_c = scale * q.k_c carries at most about
# (4 + log2(dim/4)) * 2^-24 * scale * sum_d |q_d k_cd| of rounding (a 4-term
# FMA chain and a fixed lane tree, <= 9 levels at dim 128); an error e in
# every score moves the normalised weights by at most ~2e relatively, hence
# the second term with ATTN_SCORE_TOL = 2 * 12 * 2^-24 (margin included).
# The weighted sums (<= 16 terms per lane, then a lane tree of <= 6 levels),
# the chunk merge (<= 32 chunks in sequence per wave, <= 16 wave sums in
# sequence) and exp add a few 2^-24 of max|v| (a convex combination), bounded
# by ATTN_TOL = 4e-6 at the sizes tested.
ATTN_TOL = 4e-6
ATTN_SCORE_TOL = 2 * 12 * 2.0 ** -24
# The int8 pool, gated on its dequantised rows: a lane's score sums 16
# code products in one FMA chain, then a lane tree of <= 3 levels and two
# multiplications (key scale, then scale): <= 21 roundings, 24 with margin,
# doubled as above.  The value sums take one more rounding per term (w times
# the value scale): ATTN_I8_TOL = 2 * ATTN_TOL.
ATTN_I8_TOL = 8e-6
ATTN_I8_SCORE_TOL = 2 * 24 * 2.0 ** -24


def attn_limit(q, kc, vc, ids, n_cells, scale, tol=ATTN_TOL, score_tol=ATTN_SCORE_TOL):
    """The gate above for every (query, head): an array [nq][heads]."""
    nq, heads, _ = q.shape
    lim = np.zeros((nq, heads))
    for i in range(nq):
        cells = [4 * b + e for b in ids[i] if b >= 0 for e in range(4) if 4 * b + e < n_cells]
        if not cells:
            continue
        vmax = np.abs(vc[cells].astype(np.float64)).max(axis=(0, 2))                  # [heads]
        qk = np.abs(q[i][None].astype(np.float64) * kc[cells].astype(np.float64)).sum(axis=2)
        lim[i] = vmax * (tol + score_tol * abs(scale) * qk.max(axis=0))
    return lim


SCORE_TOL = 1e-6


def score_gate(s: np.ndarray, s64: np.ndarray, tol: float = SCORE_TOL):
    """Return (ok, err_ratio) where err_ratio = max|s - s64| / (tol * max|s64|)."""
    s = np.asarray(s, dtype=np.float64)
    s64 = np.asarray(s64, dtype=np.float64)
    if s.shape != s64.shape:
        return False, float("inf")
    if s.size == 0:
        return True, 0.0
    if not np.all(np.isfinite(s)):
        return False, float("inf")
    scale = float(np.max(np.abs(s64)))
    err = float(np.max(np.abs(s - s64)))
    if scale == 0.0:
        return err == 0.0, (0.0 if err == 0.0 else float("inf"))
    ratio = err / (tol * scale)
    return ratio <= 1.0, ratio


def brute_force_topk(row, k: int) -> list[int]:
    """Selection of one row by the rank definition (quadratic; tiny rows only)."""
    row = [float(x) for x in row]
    a = len(row)
    out = [-1] * k
    for b in range(a):
        rank = sum(1 for c in range(a) if row[c] > row[b] or (row[c] == row[b] and c < b))
        if rank < k:
            out[rank] = b
    return out


def topk_invariants(scores: np.ndarray, ids: np.ndarray, k: int) -> list[str]:
    """List the violated invariants of a top-k result (empty list = valid)."""
    bad = []
    scores = np.asarray(scores)
    ids = np.asarray(ids)
    nq, a = scores.shape
    if ids.shape != (nq, k):
        return [f"shape {ids.shape} != {(nq, k)}"]
    m = min(k, a)
    for i in range(nq):
        row, sel = scores[i], ids[i]
        if np.any(sel[m:] != -1):
            bad.append(f"row {i}: padding past {m} is not -1")
        s = sel[:m]
        if np.any((s < 0) | (s >= a)):
            bad.append(f"row {i}: id out of range")
            continue
        if len(np.unique(s)) != m:
            bad.append(f"row {i}: duplicate ids")
            continue
        v = row[s].astype(np.float64)
        # rank order: score non-increasing, equal scores by increasing id
        for r in range(m - 1):
            if v[r] < v[r + 1] or (v[r] == v[r + 1] and s[r] > s[r + 1]):
                bad.append(f"row {i}: rank order broken at {r}")
                break
        if m < a:
            mask = np.ones(a, bool)
            mask[s] = False
            unsel = row[mask].astype(np.float64)
            thr = v[-1]
            if np.max(unsel) > thr:
                bad.append(f"row {i}: an unselected score beats the threshold")
            # threshold ties: every unselected block tied with the threshold must
            # have a larger id than every selected block at the threshold
            tied_unsel = np.nonzero(mask & (row.astype(np.float64) == thr))[0]
            tied_sel = s[v == thr]
            if len(tied_unsel) and len(tied_sel) and tied_unsel.min() < tied_sel.max():
                bad.append(f"row {i}: threshold ties not taken lowest-id first")
    return bad
