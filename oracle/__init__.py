"""CPU oracle for QSA block selection -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP library and its Python binding
never import it, and it imports nothing from them: the two sides share no code.

The arithmetic lives in ``qsa_oracle.c`` (plain C, gcc -O2, no fast-math) and
is reached through ``ctypes``; this module only marshals numpy arrays.

What it computes (pages: "#3108 perf(hip): optimize exact QSA block scoring and
top-k selection on gfx12", Summary items 1-2; "#337 hip: gfx12 (RDNA4) QSA
select - WMMA block scorer, prompt-aware top-k dispatch", What items 1-2):

* ``scores_f64(q, kblk, active_blocks)``: FP64 block scores
  ``s[i][b] = sum_h sum_d q[i][h][d] * kblk[b][h][d]`` for ``b < active_blocks``.
* ``topk(scores, k)``: for each row, the ids of the k largest scores, ties to
  the lower id, in rank order; slots past the row length hold -1.
* ``topk_f64(scores64, k)``: the same order on FP64 scores (diagnostic only).
* ``sparse_decode_attn_f64(q, kc, vc, ids, n_cells, scale)``: FP64 decode
  attention of each query and head over the cells of its listed blocks (page
  "#3102 perf(hip): enable wave32 QSA decode attention and MMVQ row reuse on
  gfx12", Summary item 1).
* ``sparse_decode_attn_i8_f64(q, kcode, kscale, vcode, vscale, ids, n_cells,
  scale)``: the same attention over an int8 pool (int8 codes, one binary16
  scale per cell and head; the page above, microbenchmark table, and "#3224
  [Engine] perf(hip): tune RDNA4 QSA prompt WMMA path (STRATA_HIP_WMMA stays
  opt-in)", Summary item 2).
* ``half_to_f64(bits)``: the IEEE binary16 decoding that pool uses.

Every function here is pinned by tests/test_oracle.py (hand example, exact
integer inputs, exact rationals, numpy float64 matmul, brute-force rank,
numpy lexsort, invariants).  No function here is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libqsa_oracle.so")

OK, ERR_ARG, ERR_NAN, ERR_NOMEM = 0, 1, 2, 3
_ERR_TEXT = {ERR_ARG: "bad argument", ERR_NAN: "NaN score in the active range",
             ERR_NOMEM: "out of memory"}

_lib = None


class OracleError(RuntimeError):
    pass


GCC_FLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fno-fast-math",
             "-ffp-contract=off", "-Wall", "-Wextra"]


def compile_source(src: str, out: str) -> str:
    """Compile one oracle C source into a shared library with plain gcc."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile qsa_oracle.c into oracle/libqsa_oracle.so."""
    if force or not os.path.exists(_LIB_PATH):
        compile_source(_SRC, _LIB_PATH)
    return _LIB_PATH


def _bind(path: str):
    lib = ctypes.CDLL(path)
    i64, vp = ctypes.c_int64, ctypes.c_void_p
    lib.oracle_block_scores_f64.argtypes = [vp, vp, i64, i64, i64, i64, vp]
    lib.oracle_block_scores_f64.restype = ctypes.c_int
    lib.oracle_block_topk.argtypes = [vp, i64, i64, i64, vp]
    lib.oracle_block_topk.restype = ctypes.c_int
    lib.oracle_block_topk_f64.argtypes = [vp, i64, i64, i64, vp]
    lib.oracle_block_topk_f64.restype = ctypes.c_int
    lib.oracle_sparse_decode_attn_f64.argtypes = [vp, vp, vp, vp, i64, i64, i64, i64, i64,
                                                  ctypes.c_double, vp]
    lib.oracle_sparse_decode_attn_f64.restype = ctypes.c_int
    lib.oracle_sparse_decode_attn_i8_f64.argtypes = [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                     i64, ctypes.c_double, vp]
    lib.oracle_sparse_decode_attn_i8_f64.restype = ctypes.c_int
    lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
    lib.oracle_half_to_double.restype = ctypes.c_double
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        _lib = _bind(_LIB_PATH)
    return _lib


def _check(rc: int) -> None:
    if rc != OK:
        raise OracleError(f"oracle status {rc}: {_ERR_TEXT.get(rc, 'unknown')}")


def _ptr(a: np.ndarray):
    return a.ctypes.data if a.size else None


class Oracle:
    """The oracle's three functions bound to one compiled copy of qsa_oracle.c.

    The default copy is ``oracle.default()``; tests also bind deliberately
    broken copies (mutants) to show that the pins catch plausible mistakes.
    """

    def __init__(self, lib):
        self.lib = lib

    def scores_f64(self, q: np.ndarray, kblk: np.ndarray, active_blocks: int) -> np.ndarray:
        """FP64 scores of q[nq][heads][dim] against kblk[>=active_blocks][heads][dim]."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        kblk = np.ascontiguousarray(kblk, dtype=np.float32)
        nq, heads, dim = q.shape
        if kblk.ndim != 3 or kblk.shape[1:] != (heads, dim) or kblk.shape[0] < active_blocks:
            raise ValueError("kblk must be [>=active_blocks][heads][dim]")
        out = np.empty((nq, active_blocks), dtype=np.float64)
        _check(self.lib.oracle_block_scores_f64(_ptr(q), _ptr(kblk), nq, heads, dim,
                                                active_blocks, _ptr(out)))
        return out

    def topk(self, scores: np.ndarray, k: int) -> np.ndarray:
        """Rank-ordered top-k ids (int32, -1 padded) of each row of fp32 scores."""
        scores = np.ascontiguousarray(scores, dtype=np.float32)
        nq, a = scores.shape
        ids = np.empty((nq, k), dtype=np.int32)
        _check(self.lib.oracle_block_topk(_ptr(scores), nq, a, k, _ptr(ids)))
        return ids

    def topk_f64(self, scores: np.ndarray, k: int) -> np.ndarray:
        """The same selection on FP64 scores (a diagnostic, never a gate)."""
        scores = np.ascontiguousarray(scores, dtype=np.float64)
        nq, a = scores.shape
        ids = np.empty((nq, k), dtype=np.int32)
        _check(self.lib.oracle_block_topk_f64(_ptr(scores), nq, a, k, _ptr(ids)))
        return ids

    def sparse_decode_attn_f64(self, q: np.ndarray, kc: np.ndarray, vc: np.ndarray,
                               ids: np.ndarray, n_cells: int, scale: float) -> np.ndarray:
        """FP64 attention of q[nq][heads][dim] over the cells of the blocks ids[nq][k]
        (-1 skipped) in kc/vc[cells][heads][dim], cells c < n_cells only."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        kc = np.ascontiguousarray(kc, dtype=np.float32)
        vc = np.ascontiguousarray(vc, dtype=np.float32)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        nq, heads, dim = q.shape
        if ids.ndim != 2 or ids.shape[0] != nq:
            raise ValueError("ids must be [nq][k]")
        if kc.shape[1:] != (heads, dim) or vc.shape != kc.shape or kc.shape[0] < n_cells:
            raise ValueError("kc and vc must be [>=n_cells][heads][dim]")
        out = np.empty((nq, heads, dim), dtype=np.float64)
        _check(self.lib.oracle_sparse_decode_attn_f64(_ptr(q), _ptr(kc), _ptr(vc), _ptr(ids), nq,
                                                      heads, dim, ids.shape[1], n_cells,
                                                      float(scale), _ptr(out)))
        return out

    def sparse_decode_attn_i8_f64(self, q: np.ndarray, kcode: np.ndarray, kscale: np.ndarray,
                                  vcode: np.ndarray, vscale: np.ndarray, ids: np.ndarray,
                                  n_cells: int, scale: float) -> np.ndarray:
        """FP64 attention over an int8 pool: kcode/vcode [cells][heads][dim] int8,
        kscale/vscale [cells][heads] binary16 bit patterns (uint16)."""
        q = np.ascontiguousarray(q, dtype=np.float32)
        kcode = np.ascontiguousarray(kcode, dtype=np.int8)
        vcode = np.ascontiguousarray(vcode, dtype=np.int8)
        kscale = np.ascontiguousarray(kscale, dtype=np.uint16)
        vscale = np.ascontiguousarray(vscale, dtype=np.uint16)
        ids = np.ascontiguousarray(ids, dtype=np.int32)
        nq, heads, dim = q.shape
        if ids.ndim != 2 or ids.shape[0] != nq:
            raise ValueError("ids must be [nq][k]")
        if kcode.shape[1:] != (heads, dim) or vcode.shape != kcode.shape or \
                kcode.shape[0] < n_cells or kscale.shape != kcode.shape[:2] or \
                vscale.shape != kscale.shape:
            raise ValueError("codes must be [>=n_cells][heads][dim], scales [cells][heads]")
        out = np.empty((nq, heads, dim), dtype=np.float64)
        _check(self.lib.oracle_sparse_decode_attn_i8_f64(
            _ptr(q), _ptr(kcode), _ptr(kscale), _ptr(vcode), _ptr(vscale), _ptr(ids), nq, heads,
            dim, ids.shape[1], n_cells, float(scale), _ptr(out)))
        return out

    def half_to_f64(self, bits) -> np.ndarray:
        """Values of binary16 bit patterns (any integer array), as float64."""
        b = np.asarray(bits, dtype=np.uint16)
        f = self.lib.oracle_half_to_double
        return np.array([f(int(x)) for x in b.ravel()], dtype=np.float64).reshape(b.shape)


def default() -> Oracle:
    return Oracle(_load())


def load_from(path: str) -> Oracle:
    """Bind a separately compiled copy of the oracle (used for mutant checks)."""
    return Oracle(_bind(path))


def scores_f64(q, kblk, active_blocks):
    return default().scores_f64(q, kblk, active_blocks)


def topk(scores, k):
    return default().topk(scores, k)


def topk_f64(scores, k):
    return default().topk_f64(scores, k)


def sparse_decode_attn_f64(q, kc, vc, ids, n_cells, scale):
    return default().sparse_decode_attn_f64(q, kc, vc, ids, n_cells, scale)


def sparse_decode_attn_i8_f64(q, kcode, kscale, vcode, vscale, ids, n_cells, scale):
    return default().sparse_decode_attn_i8_f64(q, kcode, kscale, vcode, vscale, ids, n_cells,
                                               scale)


def half_to_f64(bits):
    return default().half_to_f64(bits)
