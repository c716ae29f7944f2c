"""Seeded synthetic inputs for QSA block selection.

This module only draws numbers.  It holds none of the selection arithmetic
(no scores, no ordering, no top-k), so both the HIP path's tests and the CPU
oracle's tests can take their inputs from it without sharing method code.

The shapes follow the pages' workloads ("#3108 perf(hip): optimize exact QSA
block scoring and top-k selection on gfx12", Microbenchmark tables: 256 prompt
queries, one decode query, a 262,144-cell capacity; "#337 hip: gfx12 (RDNA4)
QSA select ...", What item 1: a capacity of max-context/4 + 2 blocks of 4
cells, of which only the active ones are scored).  The pages publish no input
data, seeds or test vectors; everything below is synthetic:

* q and block key summaries are N(0, 1), drawn in float64 and rounded once to
  float32, from ``numpy.random.Generator(PCG64(seed))``;
* "needle" blocks (a fraction of the active blocks) are replaced by
  ``fp32(0.8 * q[j] + 0.2 * noise)`` for a random query j, so that query's
  selection has a few clearly relevant blocks;
* the near-tie workload draws every block from 64 distinct vectors, so each
  row of scores has at most 64 + n_needle distinct values and ~1,000-way ties
  at the selection threshold;
* capacity rows past the active blocks hold quiet NaN (poison) so that a
  kernel that reads them shows it;
* the key and value cells attended after selection (``make_kv``) are N(0, 1)
  drawn directly in float32 (a cache of a quarter-million cells is too large
  to draw in float64 first), with the cells past the active blocks poisoned
  the same way.  The pages give no link between a block's summary and its
  cells that the timing would depend on, so the two are drawn independently.

Draw order per workload (fixed): q; block summaries (or the tie vectors, then
their assignment); needle block ids; needle query ids; needle noise.
"""
from __future__ import annotations

import dataclasses
import hashlib

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    nq: int            # queries per call
    heads: int
    dim: int
    active: int        # active blocks (scored and selected)
    capacity: int      # rows of the block-summary buffer (>= active)
    k: int             # blocks selected per query
    needle_frac: float = 0.0
    tie_vectors: int = 0   # > 0: every block is one of this many vectors
    poison: bool = False   # rows [active, capacity) hold quiet NaN
    seed: int = 0

    @property
    def K(self) -> int:
        return self.heads * self.dim

    @property
    def n_needles(self) -> int:
        return int(round(self.needle_frac * self.active))

    @property
    def cells(self) -> int:
        return 4 * self.active


# The five workloads: a tiny decode call, 32K and 128K prompts, a 128K decode
# call inside a 262,144-cell capacity, and a 256K near-tie prompt stress case;
# then multi-query decode at 128K (2 and 4 queries per call, the T = 2 and
# T = 4 rows of the decode table of "#3108 perf(hip): ...": speculative
# verification scores several queries against the same summaries), and one
# eighth of the 128K prompt's blocks (the share of one of 8 GPUs).
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny-decode", nq=1, heads=4, dim=64, active=512, capacity=512, k=64),
        Workload("prompt-32k", nq=256, heads=4, dim=128, active=8193, capacity=8193,
                 k=256, needle_frac=0.01),
        Workload("decode-128k", nq=1, heads=4, dim=128, active=32770, capacity=65538,
                 k=512, poison=True),
        Workload("prompt-128k", nq=256, heads=4, dim=128, active=32770, capacity=65538,
                 k=512, needle_frac=0.01, poison=True),
        Workload("prompt-256k-tie", nq=256, heads=4, dim=128, active=65538,
                 capacity=65538, k=1024, needle_frac=0.001, tie_vectors=64),
        Workload("decode-128k-t2", nq=2, heads=4, dim=128, active=32770, capacity=65538,
                 k=512, poison=True),
        Workload("decode-128k-t4", nq=4, heads=4, dim=128, active=32770, capacity=65538,
                 k=512, poison=True),
        # One GPU's share of the 128K prompt when the blocks are split over 8
        # GPUs by range: the per-shard call at its real shape.
        Workload("prompt-128k-shard8", nq=256, heads=4, dim=128, active=4097, capacity=4097,
                 k=512, needle_frac=0.01),
    ]
}

HEADLINE = "prompt-128k"


@dataclasses.dataclass
class Batch:
    workload: Workload
    q: np.ndarray            # [nq][heads][dim] float32
    kblk: np.ndarray         # [capacity][heads][dim] float32
    needle_blocks: np.ndarray  # int64 block ids that were replaced by needles
    needle_queries: np.ndarray  # int64 query id each needle was built from
    tie_assign: np.ndarray | None  # int64 vector index of each active block (tie workload)


def _normal_f32(rng: np.random.Generator, shape) -> np.ndarray:
    return rng.standard_normal(shape, dtype=np.float64).astype(np.float32)


def make_batch(w: Workload, seed: int | None = None) -> Batch:
    """Draw one batch of inputs for workload ``w`` (deterministic in the seed)."""
    rng = np.random.Generator(np.random.PCG64(w.seed if seed is None else seed))
    shape = (w.heads, w.dim)
    q = _normal_f32(rng, (w.nq,) + shape)
    kblk = np.empty((w.capacity,) + shape, dtype=np.float32)
    tie_assign = None
    if w.tie_vectors > 0:
        vecs = _normal_f32(rng, (w.tie_vectors,) + shape)
        tie_assign = rng.integers(0, w.tie_vectors, w.active)
        kblk[: w.active] = vecs[tie_assign]
    else:
        kblk[: w.active] = _normal_f32(rng, (w.active,) + shape)
    n = w.n_needles
    needle_blocks = rng.choice(w.active, n, replace=False) if n else np.zeros(0, np.int64)
    needle_queries = rng.integers(0, w.nq, n) if n else np.zeros(0, np.int64)
    if n:
        noise = rng.standard_normal((n,) + shape, dtype=np.float64)
        kblk[needle_blocks] = (0.8 * q[needle_queries].astype(np.float64) + 0.2 * noise).astype(np.float32)
    if w.capacity > w.active:
        kblk[w.active:] = np.nan if w.poison else 0.0
    return Batch(w, q, kblk, np.asarray(needle_blocks, np.int64),
                 np.asarray(needle_queries, np.int64), tie_assign)


def make_random(nq: int, heads: int, dim: int, active: int, capacity: int | None = None,
                seed: int = 0, integer: bool = False, poison: bool = True):
    """Free-shape inputs for parity cases: N(0,1) fp32, or small integers.

    With ``integer=True`` every entry is a uniform integer in [-8, 8]; with
    heads*dim <= 512 every partial sum of products stays below 2**24, so any
    fp32 summation order gives the exact result.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    capacity = active if capacity is None else capacity
    if integer:
        q = rng.integers(-8, 9, (nq, heads, dim)).astype(np.float32)
        kb = rng.integers(-8, 9, (active, heads, dim)).astype(np.float32)
    else:
        q = _normal_f32(rng, (nq, heads, dim))
        kb = _normal_f32(rng, (active, heads, dim))
    kblk = np.empty((capacity, heads, dim), dtype=np.float32)
    kblk[:active] = kb
    if capacity > active:
        kblk[active:] = np.nan if poison else 0.0
    return q, kblk


def make_kv(w: Workload, seed: int | None = None):
    """Key and value caches [4 * capacity, heads, dim] float32 for workload ``w``
    (cells of the active blocks N(0, 1), the rest quiet NaN if ``w.poison``,
    else 0).  Draw order: keys, then values, from PCG64(seed + 1)."""
    base = w.seed if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(base + 1))
    n, live = 4 * w.capacity, 4 * w.active
    out = []
    for _ in range(2):
        c = np.empty((n, w.heads, w.dim), dtype=np.float32)
        c[:live] = rng.standard_normal((live, w.heads, w.dim), dtype=np.float32)
        c[live:] = np.nan if w.poison else 0.0
        out.append(c)
    return out[0], out[1]


def make_pool_i8(cells: int, live: int, heads: int, dim: int, seed: int = 0,
                 poison: bool = True):
    """An int8 key or value pool: codes [cells, heads, dim] int8 and one
    binary16 scale per (cell, head) as uint16 bit patterns.  Codes are
    round(N(0, 40)) clipped to [-127, 127] (the spread of a quantised normal
    row), scales uniform in [0.01, 0.04] rounded to binary16.  Cells at or past
    `live` get code 0 and, with `poison`, a quiet-NaN scale (0x7E00)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    codes = np.zeros((cells, heads, dim), dtype=np.int8)
    x = np.rint(rng.standard_normal((live, heads, dim), dtype=np.float32) * 40.0)
    codes[:live] = np.clip(x, -127, 127).astype(np.int8)
    scales = np.empty((cells, heads), dtype=np.uint16)
    scales[:live] = rng.uniform(0.01, 0.04, (live, heads)).astype(np.float16).view(np.uint16)
    scales[live:] = 0x7E00 if poison else 0
    return codes, scales


def fingerprint(a: np.ndarray) -> str:
    """Content fingerprint of an array (blake2b-64 of its bytes, dtype and shape)."""
    h = hashlib.blake2b(digest_size=8)
    h.update(str(a.dtype).encode())
    h.update(str(a.shape).encode())
    h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()
