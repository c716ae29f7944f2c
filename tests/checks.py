"""Checkers shared by the oracle pins and the GPU parity tests.

These do not compute selections themselves beyond tiny brute force; they
check a result against what the definition fixes:

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
#   max_d |out - out64| <= max_c |v[c][h]| * (T + S * |scale| * max_c sum_d |q_d k_cd|)
# over the attended cells c, with T and S from attn_tols(k, dim).  A first-order
# rounding bound (u = 2^-24, every count below times u; n*u < 1e-3 throughout,
# so the second-order terms are far below the margin).  The kernels' sequences:
#
# * score of a cell (S): a lane's 4-term FMA chain (4 roundings on the first
#   product), a tree over the LPC lanes of the row (log2 LPC), the scale (1):
#   n_s = 5 + log2 LPC roundings of at most sum_d |q_d k_cd| each.  Score errors
#   up to e move the normalised weights by e relatively, on both the sum and
#   the normaliser: S = 2 * n_s * u.  int8 pool: 16 products in one chain,
#   log2 LPC, the key scale and the scale: n_s = 18 + log2 LPC.
# * T, the rest, for the worst chunk size the kernel may pick at this k (4
#   listed blocks up to k = 1024, else 8 or 16; R = 4 * CB / CPI rows per
#   lane, CPI = 64 / LPC cells per load, nch = ceil(k / CB) chunks,
#   nw = ceil(nch / 32) merge waves):
#     value sum in a chunk      R + log2 CPI   (+1 for int8: w * value scale)
#     weight sum in a chunk     R + log2 CPI
#     merge of the value sums   min(nch, 32) + nw - 1   (FMA chain per wave, then the waves in order)
#     merge of the weight sums  1 + 6 + nw - 1          (product, 64-lane tree, the waves)
#     the division              1
#     the weights themselves    2 * (2 * 2 ulp of exp + ln(4k))  (exp(s - m_j) * exp(m_j - M) as
#                               computed has relative error u*|s - M| + 2 ulps of each exp; the
#                               mean of |s - M| under the softmax weights is at most the log of
#                               the cell count; a weight error moves both sum and normaliser)
#   Each bounded against sum_c W_c |v_c| <= max|v| * sum_c W_c.  The exp
#   accuracy (2 ulp, 2^-22 relative) is the one assumption not read off the
#   kernel's own sequence.
_U = 2.0 ** -24


def _lpc(dim: int, int8: bool) -> int:
    per = 16 if int8 else 4                 # elements per lane
    lpc = 1
    while lpc * per < dim:
        lpc *= 2
    return lpc


def attn_tols(k: int, dim: int, int8: bool = False) -> tuple[float, float]:
    """(T, S) of the gate above for a call with k listed blocks and this dim."""
    import math
    lpc = _lpc(dim, int8)
    cpi = 64 // lpc
    n_s = (18 if int8 else 5) + int(math.log2(lpc))
    worst = 0.0
    for cb in ([4] if k <= 1024 else [8, 16]):
        rounds = max(1, 4 * cb // cpi)
        if rounds > 16:
            continue                        # more rows than the kernel holds: never chosen
        n_chunk = rounds + int(math.log2(cpi))
        nch = -(-max(k, 1) // cb)
        nw = -(-nch // 32)
        n = ((n_chunk + (1 if int8 else 0))   # value sums in the chunk
             + n_chunk                        # weight sums in the chunk
             + min(nch, 32) + nw - 1          # merge of the value sums
             + 1 + 6 + nw - 1                 # merge of the weight sums
             + 1                              # division
             + 2 * (2 * 4 + math.log(4 * max(k, 1))))  # the weights
        worst = max(worst, n)
    return worst * _U, 2 * n_s * _U


def attn_limit(q, kc, vc, ids, n_cells, scale, int8: bool = False):
    """The gate above for every (query, head): an array [nq][heads].  For the
    int8 pool, kc and vc are the dequantised rows (code * scale)."""
    nq, heads, dim = q.shape
    tol, score_tol = attn_tols(ids.shape[1], dim, int8)
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
