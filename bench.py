#!/usr/bin/env python3
"""Throughput of the QSA selection hot path (block scores + top-k) on one GPU.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one full selection pass over one batch of synthetic input: one
qsa_block_select call (scores, then the top-k of those scores) through the C
ABI, on the current torch stream.  Default workload: 256 prompt queries x
32,770 active blocks (a 131K context) in a 65,538-block (262,144-cell)
capacity, 4 heads x 128, k = 512.

Steps rotate over several input copies (different HBM buffers, same values) so
that the block summaries read by each step are not still sitting in the 256 MB
last-level cache from the previous one.  Inputs are resident in HBM before the
timed region starts.  Prints ONE JSON line.

Two timed passes over the same K steps:
  1. throughput: the K steps bracketed by a device synchronisation (and a HIP
     event pair) on both sides, nothing else inside -- `ms_per_step`, `value`;
  2. kernel durations: the two separate calls (qsa_block_scores,
     qsa_block_topk), each K times back to back between one HIP event pair on
     their stream -- per-stage times (kernel plus dispatch gap) and
     `roofline`.  (An event costs a few microseconds of GPU time, so no call
     carries its own.)
`roofline` reports the scorer (the dominant kernel) against the peak its
method is priced on: the algorithmic fp32 work, 2 * nq * A * heads * dim FLOP,
against the fp32 matrix-core peak (157.3 TFLOP/s) for both matrix-core
scorers; for the exact three-way bf16 split (the prompt default), which forms
six bf16 slice products per fp32 product, `bf16_pipe` beside it gives that
work (6 * 2 * nq * A * heads * dim) against the bf16 peak (2.5 PFLOP/s).  The
few-query dot-product kernel is priced on HBM (bytes of the active summaries,
the queries and the scores).

The default warmup (500 steps, about 40 ms of prompt work) is long enough for
the first timed pass to run at the settled clock: after 50 steps it read
about 7 % slower than the repeats that follow it, after 500 within 0.2 %.

Pass 1 is repeated (--repeats, default 7) and `stages.repeats` gives the
median and range of the per-step time.  For a prompt workload the same run
also times the decode call at 128K (one query, 32,770 active blocks, k = 512,
qsa_block_select) the same way: `stages.decode_select` with its HBM fraction
over the call's algorithmic bytes.  `fingerprints` are blake2b-64 digests of
the host inputs and of the outputs of the first input copy.

The CPU baseline is the CPU oracle (FP64 scores, then a sort-based top-k of its
fp32-rounded scores) on this host: scores and top-k timed apart, once on all
the threads of the host's share (the affinity set, capped by OMP_NUM_THREADS
where set) over every query row, once on one thread over a sample of rows.

With --attention (decode workloads, at most 8 queries) a step is the decode
layer's whole QSA stage: the selection above, then qsa_sparse_decode_attention
of the same queries over the cells of the selected blocks in a synthetic fp32
key/value cache of the workload's capacity (4 cells per block, rotated over the
same input copies).  `roofline_attention` then reports that call against HBM:
its algorithmic bytes are the gathered key and value rows (2 * nq * k * 4 cells
* heads * dim * 4 B; with --pool int8, dim one-byte codes and a 2-byte scale
per cell and head) plus the queries, ids and outputs, over the per-call time of
K calls replayed from a captured HIP graph between one event pair (both of its
kernels and the gap between them; launched one by one from Python, a call this
short would time the binding's host cost).  --graph
adds a pass that replays the steps from one captured HIP graph, which shows the
GPU time per step without the per-call host cost of the Python binding.
"""
from __future__ import annotations

import argparse
import concurrent.futures as cf
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from sparse_attention_kv_qsa_amd import synth  # noqa: E402

METRIC = "QSA select ms/call (score+top-k), 256q x 131K ctx; queries*blocks/s; % roofline"
UNIT = "queries*blocks/s"
# MI355X published dense peaks.
PEAK_FP32_MFMA_TFLOPS = 157.3
PEAK_BF16_MFMA_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0
# The pages' standalone figure for this workload (R9700, gfx1201): scores
# 0.65 ms + top-k 0.51 ms per call at 256 queries, 131K context.  Context only.
PAGES_SELECT_MS = 0.65 + 0.51
CSRC = os.path.join(ROOT, "sparse_attention_kv_qsa_amd", "csrc")
# Scorer kernel per precision path: (source file, counter summary under profiles/).
SCORERS = {
    "fp32": ("qsa_scores.hip", "traffic_scores_mfma_prompt-128k.txt"),
    "bf16x3": ("qsa_scores_bf16x3.hip", "traffic_scores_bf16x3_prompt-128k.txt"),
    "f16x2": ("qsa_scores_f16x2.hip", "traffic_scores_f16x2_prompt-128k.txt"),
}
# Split scorers: matrix products per fp32 product, kernel, matrix-core input type.
SPLITS = {"bf16x3": (6, "scores_bf16x3_kernel", "bf16"), "f16x2": (3, "scores_f16x2_kernel", "f16")}
# The scorer the library's AUTO mode takes for more than 8 queries.
AUTO_SPLIT = "f16x2"


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=500)
    p.add_argument("--workload", default=synth.HEADLINE, choices=list(synth.WORKLOADS))
    p.add_argument("--k", type=int, default=None,
                   help="blocks selected per query (default: the workload's k)")
    p.add_argument("--copies", type=int, default=6,
                   help="input copies rotated over the steps (defeats cache reuse)")
    p.add_argument("--scores-mode", default="auto", choices=["auto", "fp32", "bf16x3", "f16x2"],
                   help="precision mode of qsa_block_scores_ex (auto = the library default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--repeats", type=int, default=7,
                   help="timings of the K steps (median and range in stages.repeats)")
    p.add_argument("--no-decode-stage", action="store_true",
                   help="prompt workloads: skip timing the 128K decode call in the same run")
    p.add_argument("--attention", action="store_true",
                   help="decode workloads: select, then attend over the selected blocks")
    p.add_argument("--pool", default="fp32", choices=["fp32", "int8"],
                   help="--attention: key/value cells as fp32 rows, or int8 codes with one "
                        "binary16 scale per cell and head")
    p.add_argument("--graph", action="store_true",
                   help="also time the steps replayed from one captured HIP graph")
    p.add_argument("--calib-copy-mib", type=int, default=0,
                   help="only run a plain device copy of this many MiB (counter calibration)")
    return p.parse_args()


def build_digest(path: str) -> str:
    """Hash of a kernel's source file and of the library's compiler flags: the
    counters taken on a build are void once either changes."""
    import hashlib
    from sparse_attention_kv_qsa_amd.build import flags_for
    h = hashlib.sha256()
    with open(os.path.join(CSRC, path), "rb") as f:
        h.update(f.read())
    h.update(b"\0" + " ".join(flags_for(os.path.join(CSRC, path))).encode())
    return h.hexdigest()[:16]


def read_traffic(path: str, workload: str):
    """HBM bytes per scorer launch from committed counter runs, if they were
    taken on the current source and build flags of that scorer; else None."""
    src, summary = SCORERS[path]
    fname = os.path.join(ROOT, "profiles", summary)
    if workload != synth.HEADLINE or not os.path.exists(fname):
        return None
    kv = {}
    for line in open(fname):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("scorer_build_sha256_16") != build_digest(src):
        return None
    try:
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def host_threads() -> tuple[int, int]:
    """(threads of this host's share, cores in the affinity set): the affinity
    set, capped by OMP_NUM_THREADS where the host sets it (a shared GPU host
    gives each GPU's jobs that many threads)."""
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    share = min(avail, int(cap)) if cap.isdigit() and int(cap) > 0 else avail
    return max(1, share), avail


def cpu_baseline(w: synth.Workload, bt: synth.Batch, kv=None, single_rows: int = 32):
    """Time the CPU oracle: FP64 scores, then the sort-based top-k of the
    fp32-rounded scores (and with `kv`, the oracle's attention over that
    selection), each step timed on its own.  Once on every thread of the
    host's share over all query rows, once on one thread over the first
    `single_rows` rows; three passes each, medians."""
    import oracle

    orc = oracle.default()
    threads, affinity = host_threads()
    scale = 1.0 / np.sqrt(w.dim)

    def run(rows_list, pool):
        t0 = time.perf_counter()
        s64 = list(pool.map(lambda r: orc.scores_f64(bt.q[r], bt.kblk, w.active), rows_list))
        t1 = time.perf_counter()
        s32 = [a.astype(np.float32) for a in s64]
        t2 = time.perf_counter()
        ids = list(pool.map(lambda a: orc.topk(a, w.k), s32))
        t3 = time.perf_counter()
        ta = 0.0
        if kv is not None:
            def attend(args):
                r, sel = args
                if len(kv) == 4:
                    orc.sparse_decode_attn_i8_f64(bt.q[r], *kv, sel, 4 * w.active, scale)
                else:
                    orc.sparse_decode_attn_f64(bt.q[r], kv[0], kv[1], sel, 4 * w.active, scale)
            t4 = time.perf_counter()
            list(pool.map(attend, zip(rows_list, ids)))
            ta = time.perf_counter() - t4
        return t1 - t0, t3 - t2, ta

    def measure(nrows, nthreads, passes=3):
        rows_list = [r for r in np.array_split(np.arange(nrows), nthreads) if len(r)]
        with cf.ThreadPoolExecutor(nthreads) as ex:
            times = [run(rows_list, ex) for _ in range(passes)]
        ts, tk, ta = (float(np.median([t[j] for t in times])) for j in range(3))
        units = nrows * w.active
        out = {"value": units / (ts + tk + ta), "unit": UNIT, "cores": nthreads,
               "scores_value": units / ts, "topk_value": units / tk,
               "scores_ms": round(ts * 1e3, 3), "topk_ms": round(tk * 1e3, 3)}
        if kv is not None:
            out["attention_ms"] = round(ta * 1e3, 3)
        return out, passes

    allc, passes = measure(w.nq, min(threads, w.nq))
    one_rows = min(single_rows, w.nq)
    one, _ = measure(one_rows, 1)
    steps = ("FP64 scores, then the sort top-k of the fp32-rounded scores"
             + (", then FP64 attention over the selected blocks' cells" if kv else ""))
    allc.update({
        "kind": "oracle",
        "affinity_cores": affinity,
        "sample": (f"all {w.nq} queries x {w.active} blocks of {w.name} ({steps}; each step "
                   f"timed apart), {passes} passes, median; {allc['cores']} threads over query "
                   f"rows (this host's share: {threads} of {affinity} affinity cores)"),
        "single_thread": {**one, "rows": one_rows,
                          "sample": f"the first {one_rows} queries of the same batch, 1 thread, "
                                    f"{passes} passes, median"},
    })
    return allc


def graph_pass(torch, step, ncopy, K, outputs):
    """Capture one step per input copy into a HIP graph on a side stream (after
    warming the library's per-stream scratch there), replay it to cover K
    steps, and check that every replay leaves the outputs of the eager steps."""
    ref = [[t.clone() for t in group] for group in outputs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(ncopy):
            step(c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for c in range(ncopy):
            step(c)
    torch.cuda.synchronize()
    reps = max(1, K // ncopy)
    match = True
    for _ in range(3):  # replays checked one by one, eager work between them
        for group in outputs:
            for t in group:
                t.fill_(-7)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        match = match and all(torch.equal(a, b) for ga, gb in zip(outputs, ref)
                              for a, b in zip(ga, gb))
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return {"ms_per_step": round(e0.elapsed_time(e1) / (reps * ncopy), 5), "match": bool(match)}


def time_steps(torch, step, ncopy, K, repeats):
    """K steps back to back, bracketed by a device synchronisation and an
    event pair, `repeats` times.  Returns the per-step times of the first
    timing (wall clock, events) and of every repeat (wall clock), in ms."""
    out = []
    for r in range(max(1, repeats)):
        p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        p0.record()
        for it in range(K):
            step(it % ncopy)
        p1.record()
        torch.cuda.synchronize()
        out.append(((time.perf_counter() - t0) * 1e3 / K, p0.elapsed_time(p1) / K))
    return out


def spread(ms):
    return {"n": len(ms), "median_ms": round(float(np.median(ms)), 5),
            "min_ms": round(float(np.min(ms)), 5), "max_ms": round(float(np.max(ms)), 5)}


def select_bytes(w) -> float:
    """Algorithmic bytes of one select call: the active summaries and the
    queries read, the scores written and read back, the ids written."""
    return 4.0 * (w.active * w.K + w.nq * w.K + 2 * w.nq * w.active + w.nq * w.k)


def decode_stage(torch, args, ncopy):
    """The decode call at 128K in the same run: K select calls back to back
    (repeated), and the same calls replayed from a captured graph."""
    from sparse_attention_kv_qsa_amd import qsa_block_select

    wd = synth.WORKLOADS["decode-128k"]
    bt = synth.make_batch(wd)
    dev = torch.device("cuda:0")
    q = [torch.from_numpy(bt.q).to(dev) for _ in range(ncopy)]
    kb = [torch.from_numpy(bt.kblk).to(dev) for _ in range(ncopy)]
    sc = [torch.empty((wd.nq, wd.active), dtype=torch.float32, device=dev) for _ in range(ncopy)]
    ids = [torch.empty((wd.nq, wd.k), dtype=torch.int32, device=dev) for _ in range(ncopy)]

    def step(c):
        qsa_block_select(q[c], kb[c], wd.k, wd.active, scores=sc[c], ids=ids[c])

    for it in range(max(args.warmup, 2 * ncopy)):
        step(it % ncopy)
    torch.cuda.synchronize()
    K = max(args.steps, 2 * ncopy)
    reps = time_steps(torch, step, ncopy, K, args.repeats)
    wall = [r[0] for r in reps]
    graph = graph_pass(torch, step, ncopy, K, [ids, sc])
    nbytes = select_bytes(wd)
    med = float(np.median(wall)) * 1e-3
    g = graph["ms_per_step"] * 1e-3
    out = {
        "workload": (f"{wd.name}: {wd.nq} query x {wd.active} active blocks "
                     f"({wd.capacity}-block capacity), {wd.heads} heads x {wd.dim}, k={wd.k}"),
        "call": "qsa_block_select",
        "algorithmic_bytes": int(nbytes),
        "us_per_call": round(med * 1e6, 2),
        "repeats": spread(wall),
        "hbm_gbs": round(nbytes / med / 1e9, 1),
        "hbm_frac": round(nbytes / med / 1e9 / PEAK_HBM_GBS, 4),
        "graph_us_per_call": round(g * 1e6, 2),
        "graph_hbm_frac": round(nbytes / g / 1e9 / PEAK_HBM_GBS, 4),
        "graph_replays_match_eager": graph["match"],
        "target_hbm_frac": 0.60,
        "fingerprints": {"q": synth.fingerprint(bt.q), "kblk": synth.fingerprint(bt.kblk),
                         "ids": synth.fingerprint(ids[0].cpu().numpy())},
    }
    del q, kb, sc, ids
    torch.cuda.synchronize()
    return out


def main():
    args = parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the selection path "
                          "is not sharded across GPUs",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    from sparse_attention_kv_qsa_amd import (binding, qsa_block_scores_ex, qsa_block_select,
                                             qsa_block_topk, qsa_sparse_decode_attention,
                                             qsa_sparse_decode_attention_i8)

    binding.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    if args.calib_copy_mib:
        n = args.calib_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n * 4, "launches": 3}))
        return

    w = synth.WORKLOADS[args.workload]
    if args.k is not None:
        import dataclasses
        if args.k != w.k:  # a different workload: no published figure, no stored counters
            w = dataclasses.replace(w, name=f"{w.name}-k{args.k}", k=args.k)
    bt = synth.make_batch(w)
    ncopy = max(1, args.copies)
    q_d = [torch.from_numpy(bt.q).to(dev) for _ in range(ncopy)]
    k_d = [torch.from_numpy(bt.kblk).to(dev) for _ in range(ncopy)]
    s_d = [torch.empty((w.nq, w.active), dtype=torch.float32, device=dev) for _ in range(ncopy)]
    i_d = [torch.empty((w.nq, w.k), dtype=torch.int32, device=dev) for _ in range(ncopy)]
    attn = args.attention
    if attn and w.nq > 8:
        print(json.dumps({"error": "--attention times the decode layer: workloads of at most "
                          "8 queries", "workload": w.name}))
        sys.exit(2)
    n_cells = 4 * w.active
    int8 = args.pool == "int8"
    if attn and not int8:
        kv = synth.make_kv(w)
        kc_d = [torch.from_numpy(kv[0]).to(dev) for _ in range(ncopy)]
        vc_d = [torch.from_numpy(kv[1]).to(dev) for _ in range(ncopy)]
    if attn and int8:
        kq, ks = synth.make_pool_i8(4 * w.capacity, n_cells, w.heads, w.dim, seed=w.seed + 1)
        vq, vs = synth.make_pool_i8(4 * w.capacity, n_cells, w.heads, w.dim, seed=w.seed + 2)
        kv = (kq, ks, vq, vs)
        pools = [tuple(torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to(dev)
                       for a in kv) for _ in range(ncopy)]
    if attn:
        o_d = [torch.empty((w.nq, w.heads, w.dim), dtype=torch.float32, device=dev)
               for _ in range(ncopy)]
    torch.cuda.synchronize()

    mode = args.scores_mode

    def select(c):
        if mode == "auto":
            qsa_block_select(q_d[c], k_d[c], w.k, w.active, scores=s_d[c], ids=i_d[c])
        else:
            qsa_block_scores_ex(q_d[c], k_d[c], w.active, scores=s_d[c], mode=mode)
            qsa_block_topk(s_d[c], w.k, ids=i_d[c])

    def attend(c):
        if int8:
            qsa_sparse_decode_attention_i8(q_d[c], *pools[c], i_d[c], n_cells, out=o_d[c])
        else:
            qsa_sparse_decode_attention(q_d[c], kc_d[c], vc_d[c], i_d[c], n_cells, out=o_d[c])

    def step(c):
        select(c)
        if attn:
            attend(c)

    for it in range(args.warmup):
        step(it % ncopy)
    torch.cuda.synchronize()

    # Pass 1: throughput of the hot path, K steps, then repeated.
    K = args.steps
    first = time_steps(torch, step, ncopy, K, 1)[0]
    ms_step, gpu_ms_step = first
    value = w.nq * w.active / (ms_step * 1e-3)
    reps = [ms_step] + [r[0] for r in time_steps(torch, step, ncopy, K, args.repeats - 1)] \
        if args.repeats > 1 else [ms_step]

    # Pass 2: the two calls apart, each K times back to back between one
    # event pair on their stream (the kernel plus the dispatch gap to the
    # next; no per-call events, whose own cost would be counted).
    def stage_ms(call):
        return float(np.median([r[1] for r in time_steps(torch, call, ncopy, K, 3)]))

    score_ms = stage_ms(lambda c: qsa_block_scores_ex(q_d[c], k_d[c], w.active, scores=s_d[c],
                                                      mode=mode))
    topk_ms = stage_ms(lambda c: qsa_block_topk(s_d[c], w.k, ids=i_d[c]))

    attn_ms = None
    if attn:
        # Pass 2b: the attention call alone (the ids of every copy were
        # written by the passes above), K calls replayed from a captured
        # graph between one event pair.
        ga = graph_pass(torch, attend, ncopy, K, [o_d])
        attn_ms = ga["ms_per_step"]
        attn_graph_ok = ga["match"]

    graph = None
    if args.graph:
        graph = graph_pass(torch, step, ncopy, K,
                           [i_d] + ([o_d] if attn else []))

    fingerprints = {"q": synth.fingerprint(bt.q), "kblk": synth.fingerprint(bt.kblk),
                    "scores": synth.fingerprint(s_d[0].cpu().numpy()),
                    "ids": synth.fingerprint(i_d[0].cpu().numpy())}

    flop = 2.0 * w.nq * w.active * w.K  # algorithmic fp32 FLOP of the scores
    score_s = score_ms * 1e-3
    # The kernel the library runs for this shape and mode (mirrors its dispatch).
    gemv_ok = w.nq <= 8 and w.nq * -(-w.K // 256) <= 16
    if gemv_ok and mode not in SPLITS:
        path = "gemv"
    else:
        path = AUTO_SPLIT if mode == "auto" else mode
    if path == "gemv":
        nbytes = 4.0 * (w.active * w.K + w.nq * w.K + w.nq * w.active)
        gbs = nbytes / score_s / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": "scores_gemv_kernel", "bytes_per_launch": int(nbytes),
                "ms_per_launch": round(score_ms, 5)}
    else:
        tf = flop / score_s / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP32_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
                "traffic": read_traffic(path, w.name),
                "kernel": "scores_mfma_kernel" if path == "fp32" else SPLITS[path][1],
                "flop_per_launch": int(flop), "ms_per_launch": round(score_ms, 5)}
        if path in SPLITS:
            # The split forms n bf16 (fp16) piece products per fp32 product;
            # both have the same dense matrix-core peak.
            n, _, ty = SPLITS[path]
            roof[f"{ty}_pipe"] = {"achieved": round(n * tf, 2), "peak": PEAK_BF16_MFMA_TFLOPS,
                                  "unit": "TFLOP/s", "frac": round(n * tf / PEAK_BF16_MFMA_TFLOPS, 4),
                                  "flop_per_launch": int(n * flop)}
    topk_bytes = 4.0 * (w.nq * w.active + w.nq * w.k)
    sbytes = select_bytes(w)

    out = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": UNIT,
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": (round(value / (256 * 32770 / (PAGES_SELECT_MS * 1e-3)), 3)
                        if w.name == synth.HEADLINE else None),
        "dtype": path if path in SPLITS else "f32",
        "data": "synthetic (seeded N(0,1) fp32 queries and block summaries, planted needles)",
        "config": {
            "workload": (f"{w.name}: {w.nq} queries x {w.active} active blocks "
                         f"({w.capacity}-block capacity), {w.heads} heads x {w.dim}, k={w.k}"),
            "nq": w.nq, "active_blocks": w.active, "capacity_blocks": w.capacity,
            "heads": w.heads, "dim": w.dim, "k": w.k, "input_copies": ncopy,
            "scores_mode": mode, "step": "qsa_block_select" if mode == "auto" else
            "qsa_block_scores_ex + qsa_block_topk",
        },
        "stages": {
            "gpu_ms_per_step": round(gpu_ms_step, 5),
            "repeats": spread(reps),
            "step_hbm_gbs": round(sbytes / (ms_step * 1e-3) / 1e9, 1),
            "step_hbm_frac": round(sbytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scores_ms": round(score_ms, 5),
            "topk_ms": round(topk_ms, 5),
            "stage_timing": "each call K times back to back between one event pair, median of 3",
            "topk_gbs": round(topk_bytes / (topk_ms * 1e-3) / 1e9, 1),
            "topk_hbm_frac": round(topk_bytes / (topk_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scores_kernel": path,
        },
        "roofline": roof,
        "fingerprints": fingerprints,
        "cpu_baseline": None,
    }
    if graph is not None:
        out["stages"]["graph_ms_per_step"] = graph["ms_per_step"]
        out["stages"]["graph_replays_match_eager"] = graph["match"]
    if attn:
        # Algorithmic bytes of one attention call: the gathered key and value
        # rows, the queries, the ids and the outputs.
        gathered = (2.0 * w.nq * w.k * 4 * (w.K + 2 * w.heads) if int8 else
                    2.0 * w.nq * w.k * 4 * w.K * 4)
        abytes = gathered + 4.0 * (2 * w.nq * w.K + w.nq * w.k)
        gbs = abytes / (attn_ms * 1e-3) / 1e9
        out["metric"] = ("QSA decode layer: select + block-sparse attention over the "
                         "selected blocks; queries*blocks/s")
        out["vs_baseline"] = None
        out["config"]["step"] += " + qsa_sparse_decode_attention"
        out["config"]["kv_cells"] = 4 * w.capacity
        out["config"]["attended_cells"] = 4 * w.k
        out["config"]["kv_pool"] = args.pool
        out["data"] += ("; int8 key/value codes round(N(0,40)) with binary16 scales in "
                        "[0.01, 0.04], NaN scales past the active blocks" if int8 else
                        "; N(0,1) fp32 key/value cells, NaN past the active blocks")
        out["stages"]["attention_ms"] = round(attn_ms, 5)
        out["stages"]["attention_graph_replays_match_eager"] = attn_graph_ok
        out["roofline_attention"] = {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
            "bytes_per_call": int(abytes),
            "kernel": ("attn_chunk_i8_kernel" if int8 else "attn_chunk_kernel")
            + " + attn_merge_kernel (one call)"}
    if w.nq > 8 and not attn and not args.no_decode_stage:
        del s_d, i_d
        out["stages"]["decode_select"] = decode_stage(torch, args, ncopy)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, bt, kv if attn else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
