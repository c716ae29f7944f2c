"""qsa_block_select_noalloc through the C ABI against qsa_block_select.

The allocation-free entry point runs the same kernels with its scratch in a
static device array; its scores and ids must equal qsa_block_select's
bitwise.  Two calls in a row share the array, the second with a smaller
input, so a stale word left by the first call would show.  Shapes cover the
fused decode select (scratch for the published group words), the few-row
top-k after a separate scorer (256-element groups), a prompt batch (no
scratch) and a heavy-tie decode row.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from sparse_attention_kv_qsa_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sparse_attention_kv_qsa_amd import binding
    return binding.load_library()


def c_select(lib, entry, q, kb, active, k):
    nq, heads, dim = q.shape
    s = torch.full((nq, active), -5.0, dtype=torch.float32, device=q.device)
    ids = torch.full((nq, k), -7, dtype=torch.int32, device=q.device)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream or None)
    st = getattr(lib, entry)(q.data_ptr(), kb.data_ptr(), nq, heads, dim, active, k,
                             s.data_ptr(), ids.data_ptr(), stream)
    assert st == 0, f"{entry}: status {st}"
    return s, ids


def inputs(nq, heads, dim, active, seed, ties=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((nq, heads, dim)).astype(np.float32)
    if ties:
        vecs = rng.standard_normal((ties, heads, dim)).astype(np.float32)
        kb = vecs[rng.integers(0, ties, active + 3)]
    else:
        kb = rng.standard_normal((active + 3, heads, dim)).astype(np.float32)
    kb[active:] = np.nan  # rows past the active blocks are never read
    return torch.from_numpy(q).cuda(), torch.from_numpy(np.ascontiguousarray(kb)).cuda()


PAIRS = [  # (first call, second smaller call): (nq, heads, dim, active, k, ties)
    ((1, 4, 128, 32770, 512, 0), (1, 4, 128, 5000, 100, 0)),       # fused decode select
    ((4, 4, 128, 32770, 2048, 0), (2, 4, 64, 700, 64, 0)),          # more published words first
    ((2, 4, 64, 300000, 512, 0), (1, 4, 64, 140000, 64, 0)),        # scorer + 256-element groups
    ((1, 4, 128, 32770, 512, 7), (1, 4, 128, 2049, 300, 5)),        # mass ties: fallback path
    ((256, 4, 128, 8193, 256, 0), (40, 4, 128, 2000, 100, 0)),      # prompt batch: no scratch
]


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_select(lib, first, second):
    for n, shape in enumerate((first, second)):
        nq, heads, dim, active, k, ties = shape
        print(f"\n[noalloc] call {n}: nq={nq} K={heads * dim} A={active} k={k} ties={ties}",
              flush=True)
        q, kb = inputs(nq, heads, dim, active, seed=active + k + n, ties=ties)
        s_ref, ids_ref = c_select(lib, "qsa_block_select", q, kb, active, k)
        s_na, ids_na = c_select(lib, "qsa_block_select_noalloc", q, kb, active, k)
        torch.cuda.synchronize()
        assert torch.equal(s_na, s_ref), "scores differ"
        assert torch.equal(ids_na, ids_ref), "ids differ"
        assert torch.all(ids_na[:, : min(k, active)] >= 0)


def test_noalloc_edges(lib):
    q, kb = inputs(3, 4, 64, 100, seed=1)
    s, ids = c_select(lib, "qsa_block_select_noalloc", q, kb, 0, 5)   # no active block
    torch.cuda.synchronize()
    assert torch.all(ids == -1)
    s, ids = c_select(lib, "qsa_block_select_noalloc", q, kb, 100, 0)  # scores only
    s_ref, _ = c_select(lib, "qsa_block_select", q, kb, 100, 0)
    torch.cuda.synchronize()
    assert torch.equal(s, s_ref)


def test_noalloc_first_call_captured_in_a_graph(lib):
    """The allocation-free select needs no warm-up call before capture: the
    first call on a fresh stream goes straight into a HIP graph.  Three
    replays, with eager library work and synchronisations between them, each
    reproduce the eager results bitwise."""
    from sparse_attention_kv_qsa_amd import qsa_block_select, qsa_block_select_noalloc
    shapes = [(1, 4, 128, 32770, 512), (2, 4, 64, 300000, 256)]  # fused decode; scorer + groups of 256
    ins, outs, refs = [], [], []
    for n, (nq, heads, dim, active, k) in enumerate(shapes):
        q, kb = inputs(nq, heads, dim, active, seed=40 + n)
        ins.append((q, kb, active, k))
        outs.append((torch.empty((nq, active), dtype=torch.float32, device="cuda"),
                     torch.empty((nq, k), dtype=torch.int32, device="cuda")))
        refs.append(qsa_block_select(q, kb, k, active))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        for (q, kb, active, k), (s, ids) in zip(ins, outs):
            qsa_block_select_noalloc(q, kb, k, active, scores=s, ids=ids)
    torch.cuda.synchronize()
    for rep in range(3):
        for s, ids in outs:
            s.fill_(-3.0)
            ids.fill_(-9)
        q, kb, active, k = ins[1]
        qsa_block_select_noalloc(q, kb, 17, 5000)   # eager work sharing the static scratch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (s, ids), (s_ref, ids_ref) in zip(outs, refs):
            assert torch.equal(s, s_ref) and torch.equal(ids, ids_ref), f"replay {rep}"
