"""GPU parity of the block-sparse decode attention (through the C ABI) against
the CPU oracle's FP64 attention.

Gate, the same formula at every size: for every query i and head h,
    max_d |out_gpu[i][h][d] - out64[i][h][d]| <= attn_limit(...)[i][h]
= max|v| of the attended cells x (T + S x scale x max_c sum_d |q_d k_cd|), where
T(k, dim) and S(dim) are a first-order rounding bound over the kernels' own
sequences (chunk sums, merge chains, exp, division; tests/checks.py derives
them: T is 2.4e-6 to 8.3e-6 for k = 1 ... 4096 at dim 128), bitwise where the
exact result is an fp32 number (a single attended cell, no attended cell).  The
int8 pool is gated the same way on its dequantised rows (code * binary16
scale, exact in fp32) with the int8 kernel's sequences.  The attended cells of
a query are those of its listed blocks (4 per block) below n_cells.
"""
from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from checks import attn_limit
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


def gpu_attn(q, kc, vc, ids, n_cells, scale):
    from sparse_attention_kv_qsa_amd import qsa_sparse_decode_attention
    out = qsa_sparse_decode_attention(torch.from_numpy(q).cuda(), torch.from_numpy(kc).cuda(),
                                      torch.from_numpy(vc).cuda(),
                                      torch.from_numpy(np.ascontiguousarray(ids, np.int32)).cuda(),
                                      n_cells, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_attn(q, kc, vc, ids, n_cells, scale):
    got = gpu_attn(q, kc, vc, ids, n_cells, scale)
    want = ORC.sparse_decode_attn_f64(q, kc, vc, ids, n_cells, scale)
    err = np.abs(got.astype(np.float64) - want).max(axis=2)        # [nq][heads]
    lim = attn_limit(q, kc, vc, ids, n_cells, scale)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{len(bad)} (query, head) pairs over the gate; first {tuple(bad[0])}: "
                           f"error {err[tuple(bad[0])]:.3e} vs limit {lim[tuple(bad[0])]:.3e}")
    return got


def case(seed, nq, heads, dim, n_cells, k, cap_extra=5, pad=0.0, dup=False, past=False):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((nq, heads, dim)).astype(np.float32)
    kc = rng.standard_normal((n_cells + cap_extra, heads, dim)).astype(np.float32)
    vc = rng.standard_normal((n_cells + cap_extra, heads, dim)).astype(np.float32)
    kc[n_cells:] = np.nan  # never read
    vc[n_cells:] = np.nan
    nblocks = (n_cells + 3) // 4
    ids = np.stack([rng.choice(nblocks, size=k, replace=k > nblocks) for _ in range(nq)]).astype(np.int32) \
        if k else np.zeros((nq, 0), np.int32)
    if pad and k:
        ids[rng.random(ids.shape) < pad] = -1
    if dup and k >= 2:
        ids[:, 1] = ids[:, 0]
    if past and k >= 3:
        ids[:, 2] = nblocks + 7  # a block wholly past n_cells: skipped
    return q, kc, vc, ids


SHAPES = [  # nq, heads, dim, n_cells, k
    (1, 4, 128, 2048, 512), (1, 4, 128, 4001, 300), (2, 4, 128, 1000, 64), (4, 4, 128, 9000, 512),
    (1, 1, 4, 37, 9), (3, 2, 8, 50, 13), (1, 3, 16, 99, 25), (2, 2, 32, 130, 7), (1, 8, 64, 513, 8),
    (2, 2, 96, 300, 17), (8, 4, 128, 600, 129), (1, 2, 128, 5, 1), (3, 4, 64, 257, 33),
    # chunks of 8 blocks (k > 1024), and of 16 (more than 4096 chunk waves, dim <= 64)
    (1, 4, 128, 20000, 2000), (1, 4, 128, 17000, 3000), (2, 2, 64, 17000, 4096),
    (3, 4, 64, 17000, 3000), (5, 4, 128, 17000, 2000),
    # the chunk-size boundaries: 256 chunks of 4 blocks, 129 of 8
    (1, 4, 128, 9000, 1024), (1, 4, 128, 9000, 1025),
]


@pytest.mark.parametrize("nq,heads,dim,n_cells,k", SHAPES)
def test_attention_random(nq, heads, dim, n_cells, k):
    q, kc, vc, ids = case(nq * 31 + dim + k, nq, heads, dim, n_cells, k, pad=0.1, dup=True, past=True)
    check_attn(q, kc, vc, ids, n_cells, 1.0 / np.sqrt(dim))


def test_attention_scales_and_large_scores():
    q, kc, vc, ids = case(5, 2, 4, 128, 800, 64)
    for scale in (0.0, 0.01, 1.0 / np.sqrt(128), 1.0, 8.0):   # scale 8: scores in the hundreds
        check_attn(q, kc, vc, ids, 800, scale)


def test_attention_single_cell_and_empty_are_exact():
    q, kc, vc, _ = case(6, 2, 3, 64, 41, 0)
    one = np.array([[10, -1], [-1, 10]], np.int32)   # block 10: cells 40 (valid), 41-43 (past n_cells)
    got = gpu_attn(q, kc, vc, one, 41, 0.3)
    assert np.array_equal(got[0], vc[40]) and np.array_equal(got[1], vc[40])
    empty = np.full((2, 4), -1, np.int32)
    assert np.all(gpu_attn(q, kc, vc, empty, 41, 0.3) == 0)
    assert np.all(gpu_attn(q, kc, vc, np.zeros((2, 0), np.int32), 41, 0.3) == 0)


def test_attention_deterministic_and_order_insensitive():
    q, kc, vc, ids = case(7, 2, 4, 128, 3000, 256)
    a = gpu_attn(q, kc, vc, ids, 3000, 0.1)
    assert np.array_equal(a, gpu_attn(q, kc, vc, ids, 3000, 0.1))
    b = check_attn(q, kc, vc, ids[:, ::-1].copy(), 3000, 0.1)
    lim = attn_limit(q, kc, vc, ids, 3000, 0.1)[..., None]
    assert np.all(np.abs(a.astype(np.float64) - b) <= 2 * lim)


def test_attention_after_selection():
    """The decode chain: scores, top-k, then attention over the selected blocks."""
    from sparse_attention_kv_qsa_amd import qsa_block_select
    w = synth.WORKLOADS["tiny-decode"]
    bt = synth.make_batch(w)
    rng = np.random.default_rng(8)
    n_cells = 4 * w.active - 1                       # a partial last block
    kc = rng.standard_normal((4 * w.capacity, w.heads, w.dim)).astype(np.float32)
    vc = rng.standard_normal((4 * w.capacity, w.heads, w.dim)).astype(np.float32)
    _, ids = qsa_block_select(torch.from_numpy(bt.q).cuda(), torch.from_numpy(bt.kblk).cuda(), w.k,
                              w.active)
    ids = ids.cpu().numpy()
    check_attn(bt.q, kc, vc, ids, n_cells, 1.0 / np.sqrt(w.dim))


@pytest.mark.parametrize("name", ["decode-128k", "decode-128k-t4"])
def test_attention_full_size_after_selection(name):
    """The benchmarked decode layer at full size: a 262,152-cell fp32 cache, the
    ids of the library's own selection, every output checked."""
    from sparse_attention_kv_qsa_amd import qsa_block_select
    w = synth.WORKLOADS[name]
    bt = synth.make_batch(w)
    kc, vc = synth.make_kv(w)
    _, ids = qsa_block_select(torch.from_numpy(bt.q).cuda(), torch.from_numpy(bt.kblk).cuda(), w.k,
                              w.active)
    check_attn(bt.q, kc, vc, ids.cpu().numpy(), 4 * w.active, 1.0 / np.sqrt(w.dim))


# ------------------------------------------------------------ int8 pool ----

def dequantize(codes, scale_bits):
    return codes.astype(np.float32) * scale_bits.view(np.float16).astype(np.float32)[..., None]


def gpu_attn_i8(q, kq, ks, vq, vs, ids, n_cells, scale):
    from sparse_attention_kv_qsa_amd import qsa_sparse_decode_attention_i8
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    out = qsa_sparse_decode_attention_i8(t(q), t(kq), t(ks.view(np.int16)), t(vq),
                                         t(vs.view(np.int16)), t(ids.astype(np.int32)),
                                         n_cells, scale)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_attn_i8(q, kq, ks, vq, vs, ids, n_cells, scale):
    got = gpu_attn_i8(q, kq, ks, vq, vs, ids, n_cells, scale)
    want = ORC.sparse_decode_attn_i8_f64(q, kq, ks, vq, vs, ids, n_cells, scale)
    err = np.abs(got.astype(np.float64) - want).max(axis=2)
    lim = attn_limit(q, dequantize(kq, ks), dequantize(vq, vs), ids, n_cells, scale, int8=True)
    bad = np.argwhere(err > lim)
    assert bad.size == 0, (f"{len(bad)} (query, head) pairs over the gate; first {tuple(bad[0])}: "
                           f"error {err[tuple(bad[0])]:.3e} vs limit {lim[tuple(bad[0])]:.3e}")
    return got


def case_i8(seed, nq, heads, dim, n_cells, k, cap_extra=5, pad=0.0, dup=False, past=False):
    q, _, _, ids = case(seed, nq, heads, dim, n_cells, k, cap_extra, pad, dup, past)
    kq, ks = synth.make_pool_i8(n_cells + cap_extra, n_cells, heads, dim, seed=seed + 1)
    vq, vs = synth.make_pool_i8(n_cells + cap_extra, n_cells, heads, dim, seed=seed + 2)
    return q, kq, ks, vq, vs, ids  # scales past n_cells are NaN: never read


SHAPES_I8 = [  # nq, heads, dim, n_cells, k
    (1, 4, 128, 2048, 512), (1, 4, 128, 4001, 300), (4, 4, 128, 9000, 512), (1, 1, 16, 37, 9),
    (3, 2, 32, 130, 13), (1, 3, 48, 99, 25), (2, 8, 64, 513, 8), (2, 2, 80, 300, 17),
    (8, 4, 96, 600, 129), (1, 2, 112, 5, 1), (3, 4, 128, 257, 33),
    # chunks of 8 blocks (k > 1024), and of 16 (more than 4096 chunk waves)
    (1, 4, 128, 20000, 2000), (2, 4, 128, 17000, 4096), (1, 2, 48, 9000, 2049),
    (3, 4, 128, 17000, 4096), (9, 2, 64, 9000, 2000),
]


@pytest.mark.parametrize("nq,heads,dim,n_cells,k", SHAPES_I8)
def test_attention_i8_random(nq, heads, dim, n_cells, k):
    q, kq, ks, vq, vs, ids = case_i8(nq * 37 + dim + k, nq, heads, dim, n_cells, k, pad=0.1,
                                     dup=True, past=True)
    check_attn_i8(q, kq, ks, vq, vs, ids, n_cells, 1.0 / np.sqrt(dim))


def test_attention_i8_scales_extreme_codes():
    q, kq, ks, vq, vs, ids = case_i8(9, 2, 4, 128, 800, 64)
    kq[:800:3] = 127
    vq[1:800:5] = -127
    kq[2:800:7, :, ::2] = -128          # the one code without a positive twin
    for scale in (0.0, 0.05, 1.0 / np.sqrt(128), 1.0):
        check_attn_i8(q, kq, ks, vq, vs, ids, 800, scale)


def test_attention_i8_single_cell_and_empty_are_exact():
    q, kq, ks, vq, vs, _ = case_i8(10, 2, 3, 64, 41, 0)
    vq[40, 1, :3] = [-128, 127, 0]
    one = np.array([[10, -1], [-1, 10]], np.int32)
    got = gpu_attn_i8(q, kq, ks, vq, vs, one, 41, 0.3)
    want = dequantize(vq, vs)[40]
    assert np.array_equal(got[0], want) and np.array_equal(got[1], want)
    assert np.all(gpu_attn_i8(q, kq, ks, vq, vs, np.full((2, 4), -1, np.int32), 41, 0.3) == 0)


def test_attention_i8_full_size_after_selection():
    """decode-128k on an int8 pool of 262,152 cells: the library's selection,
    then attention over it, every output checked."""
    from sparse_attention_kv_qsa_amd import qsa_block_select
    w = synth.WORKLOADS["decode-128k"]
    bt = synth.make_batch(w)
    cells = 4 * w.capacity
    kq, ks = synth.make_pool_i8(cells, 4 * w.active, w.heads, w.dim, seed=11)
    vq, vs = synth.make_pool_i8(cells, 4 * w.active, w.heads, w.dim, seed=12)
    _, ids = qsa_block_select(torch.from_numpy(bt.q).cuda(), torch.from_numpy(bt.kblk).cuda(), w.k,
                              w.active)
    check_attn_i8(bt.q, kq, ks, vq, vs, ids.cpu().numpy(), 4 * w.active, 1.0 / np.sqrt(w.dim))


@pytest.mark.parametrize("nq,active,k", [(1, 5000, 256), (3, 20000, 1024), (20, 3000, 100)])
def test_decode_layer_replays_from_a_graph(nq, active, k):
    """Select then attention (both pools) captured into one HIP graph on a side
    stream: every replay, with eager library calls and synchronisations
    between replays, reproduces the eager outputs bitwise.  (nq = 20 takes
    the one-workgroup-per-row top-k, the others the whole-GPU one.)"""
    from sparse_attention_kv_qsa_amd import (qsa_block_select, qsa_sparse_decode_attention,
                                             qsa_sparse_decode_attention_i8)
    heads, dim = 4, 64
    q, kb = synth.make_random(nq, heads, dim, active, capacity=active + 2, seed=active + nq)
    rng = np.random.default_rng(nq)
    cells = 4 * (active + 2)
    kc = rng.standard_normal((cells, heads, dim)).astype(np.float32)
    vc = rng.standard_normal((cells, heads, dim)).astype(np.float32)
    kq, ks = synth.make_pool_i8(cells, 4 * active, heads, dim, seed=3)
    vq, vs = synth.make_pool_i8(cells, 4 * active, heads, dim, seed=4)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
    qd, kbd, kcd, vcd = t(q), t(kb), t(kc), t(vc)
    pool = (t(kq), t(ks.view(np.int16)), t(vq), t(vs.view(np.int16)))
    scores = torch.empty((nq, active), dtype=torch.float32, device="cuda")
    ids = torch.empty((nq, k), dtype=torch.int32, device="cuda")
    out = torch.empty((nq, heads, dim), dtype=torch.float32, device="cuda")
    out8 = torch.empty_like(out)

    def layer():
        qsa_block_select(qd, kbd, k, active, scores=scores, ids=ids)
        qsa_sparse_decode_attention(qd, kcd, vcd, ids, 4 * active, out=out)
        qsa_sparse_decode_attention_i8(qd, *pool, ids, 4 * active, out=out8)

    layer()
    torch.cuda.synchronize()
    want = [x.clone() for x in (scores, ids, out, out8)]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        layer()  # the library's scratch for this stream is allocated here, not in the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        layer()
    torch.cuda.synchronize()
    other = t(synth.make_random(nq, heads, dim, active, capacity=active + 2, seed=99)[0])
    for rep in range(3):
        for x in (scores, ids, out, out8):
            x.fill_(-3)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, y in zip(("scores", "ids", "out", "out8"), (scores, ids, out, out8), want):
            assert torch.equal(x, y), f"replay {rep}: {name} differs from the eager result"
        # eager work on the default stream between replays
        qsa_block_select(other, kbd, k, active)
        torch.cuda.synchronize()
    # the eager outputs are still the expected ones after the replays
    check_attn(q, kc, vc, want[1].cpu().numpy(), 4 * active, 1.0 / np.sqrt(dim))


def test_decode_layers_on_concurrent_streams():
    """Three decode layers (select, then attention over the selected cells)
    enqueued interleaved on three streams, with no synchronisation between
    them: each stream has its own library scratch, so every stream's results
    equal those of the same layer run alone on the default stream."""
    from sparse_attention_kv_qsa_amd import qsa_block_select, qsa_sparse_decode_attention
    rng = np.random.default_rng(77)
    layers = []
    for nq, active, k in [(1, 32770, 512), (2, 20000, 300), (4, 9000, 1024)]:
        q = torch.from_numpy(rng.standard_normal((nq, 4, 128)).astype(np.float32)).cuda()
        kb = torch.from_numpy(rng.standard_normal((active, 4, 128)).astype(np.float32)).cuda()
        kc = torch.from_numpy(rng.standard_normal((4 * active, 4, 128)).astype(np.float32)).cuda()
        vc = torch.from_numpy(rng.standard_normal((4 * active, 4, 128)).astype(np.float32)).cuda()
        layers.append((q, kb, kc, vc, active, k))

    def run(layer):
        q, kb, kc, vc, active, k = layer
        s, ids = qsa_block_select(q, kb, k, active)
        return s, ids, qsa_sparse_decode_attention(q, kc, vc, ids, 4 * active)

    refs = [run(layer) for layer in layers]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in layers]
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    results = [None] * len(layers)
    for rep in range(3):
        for i, (st, layer) in enumerate(zip(streams, layers)):
            with torch.cuda.stream(st):
                results[i] = run(layer)
    torch.cuda.synchronize()
    for got, want in zip(results, refs):
        for a, b in zip(got, want):
            assert torch.equal(a, b)
