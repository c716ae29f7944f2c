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
  2. kernel durations: the same steps as the two separate calls
     (qsa_block_scores, qsa_block_topk) with HIP events recorded on their
     stream around each -- per-stage times and `roofline`.  (An event costs
     a few microseconds of GPU time, so pass 1 carries none.)
`roofline` reports the scorer (the dominant kernel) against the peak of the
unit it runs on: fp32 MFMA with 2 * nq * A * heads * dim FLOP; bf16 MFMA on the
exact three-way split (the prompt default), whose method forms six bf16 slice
products per fp32 product (6 * 2 * nq * A * heads * dim FLOP), with the
fp32-equivalent rate beside it; or HBM for the few-query dot-product kernel
(bytes of the active summaries, the queries and the scores).

The CPU baseline is the CPU oracle (FP64 scores, then a sort-based top-k of its
fp32-rounded scores) timed on this host's cores over the same workload.

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
}


def parse_args():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--workload", default=synth.HEADLINE, choices=list(synth.WORKLOADS))
    p.add_argument("--k", type=int, default=None,
                   help="blocks selected per query (default: the workload's k)")
    p.add_argument("--copies", type=int, default=6,
                   help="input copies rotated over the steps (defeats cache reuse)")
    p.add_argument("--scores-mode", default="auto", choices=["auto", "fp32", "bf16x3"],
                   help="precision mode of qsa_block_scores_ex (auto = the library default)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-threads", type=int, default=16)
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


def source_digest(path: str) -> str:
    """Hash of a kernel's source file (the counters are void once it changes)."""
    import hashlib
    with open(os.path.join(CSRC, path), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic(path: str, workload: str):
    """HBM bytes per scorer launch from committed counter runs, if they were
    taken on the current source of that scorer; else None."""
    src, summary = SCORERS[path]
    fname = os.path.join(ROOT, "profiles", summary)
    if workload != synth.HEADLINE or not os.path.exists(fname):
        return None
    kv = {}
    for line in open(fname):
        if ":" in line and not line.startswith("#"):
            key, val = line.split(":", 1)
            kv[key.strip()] = val.strip()
    if kv.get("scorer_source_sha256_16") != source_digest(src):
        return None
    try:
        return int(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w: synth.Workload, bt: synth.Batch, threads: int, kv=None):
    """Time the CPU oracle on all queries of the workload, `passes` times (with
    `kv` = (keys, values): the oracle's attention over its own selection too)."""
    import oracle

    orc = oracle.default()
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    threads = max(1, min(threads, avail or 1))
    chunks = np.array_split(np.arange(w.nq), threads)

    def run(rows):
        if len(rows) == 0:
            return
        s64 = orc.scores_f64(bt.q[rows], bt.kblk, w.active)
        ids = orc.topk(s64.astype(np.float32), w.k)
        if kv is not None and len(kv) == 4:
            orc.sparse_decode_attn_i8_f64(bt.q[rows], *kv, ids, 4 * w.active,
                                          1.0 / np.sqrt(w.dim))
        elif kv is not None:
            orc.sparse_decode_attn_f64(bt.q[rows], kv[0], kv[1], ids, 4 * w.active,
                                       1.0 / np.sqrt(w.dim))

    passes, rates = 3, []
    with cf.ThreadPoolExecutor(threads) as ex:
        for _ in range(passes):
            t0 = time.perf_counter()
            list(ex.map(run, chunks))
            dt = time.perf_counter() - t0
            rates.append(w.nq * w.active / dt)
    return {
        "value": float(np.median(rates)),
        "unit": UNIT,
        "cores": threads,
        "kind": "oracle",
        "sample": (f"all {w.nq} queries x {w.active} blocks of {w.name} (FP64 scores + sort "
                   f"top-k of the fp32-rounded scores"
                   + (", then FP64 attention over the selected blocks' cells" if kv else "")
                   + f"), {passes} passes, median; {threads} threads over query rows"),
    }


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

    # Pass 1: throughput of the hot path.
    K = args.steps
    p0, p1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    p0.record()
    for it in range(K):
        step(it % ncopy)
    p1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / K
    value = w.nq * w.active / (wall / K)
    gpu_ms_step = p0.elapsed_time(p1) / K

    # Pass 2: per-kernel durations, events around the two separate calls.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
    torch.cuda.synchronize()
    for it in range(K):
        c = it % ncopy
        e0, e1, e2 = ev[it]
        e0.record()
        qsa_block_scores_ex(q_d[c], k_d[c], w.active, scores=s_d[c], mode=mode)
        e1.record()
        qsa_block_topk(s_d[c], w.k, ids=i_d[c])
        e2.record()
    torch.cuda.synchronize()
    score_ms = [ev[i][0].elapsed_time(ev[i][1]) for i in range(K)]
    topk_ms = [ev[i][1].elapsed_time(ev[i][2]) for i in range(K)]

    attn_ms = None
    if attn:
        # Pass 2b: the attention call alone (the ids of every copy were
        # written by the passes above), K calls replayed from a captured
        # graph between one event pair: the per-call time on the stream, both
        # kernels and the gap between them included.  Launched one by one
        # from Python, a call this short would time the binding's host cost
        # instead; an event pair per call would add its own microseconds.
        ga = graph_pass(torch, attend, ncopy, K, [o_d])
        attn_ms = [ga["ms_per_step"]]
        attn_graph_ok = ga["match"]

    graph = None
    if args.graph:
        graph = graph_pass(torch, step, ncopy, K,
                           [i_d] + ([o_d] if attn else []))

    flop = 2.0 * w.nq * w.active * w.K  # fp32-equivalent FLOP of the scores
    score_avg_s = float(np.mean(score_ms)) * 1e-3
    # The kernel the library runs for this shape and mode (mirrors its dispatch).
    gemv_ok = w.nq <= 8 and w.nq * -(-w.K // 256) <= 16
    if gemv_ok and mode != "bf16x3":
        path = "gemv"
    else:
        path = "bf16x3" if mode in ("auto", "bf16x3") else "fp32"
    extra = {}
    select_bytes = 4.0 * (w.active * w.K + w.nq * w.K + 2 * w.nq * w.active + w.nq * w.k)
    if path == "gemv":
        nbytes = 4.0 * (w.active * w.K + w.nq * w.K + w.nq * w.active)
        gbs = nbytes / score_avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                "kernel": "scores_gemv_kernel"}
    elif path == "fp32":
        tf = flop / score_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_FP32_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / PEAK_FP32_MFMA_TFLOPS, 4),
                "traffic": read_traffic("fp32", w.name), "kernel": "scores_mfma_kernel"}
    else:
        # The split method forms six bf16 slice products per fp32 product: its
        # algorithmic work on the bf16 matrix cores is 6 * 2 * nq * A * K.
        tf = 6.0 * flop / score_avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_MFMA_TFLOPS,
                "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_MFMA_TFLOPS, 4),
                "traffic": read_traffic("bf16x3", w.name), "kernel": "scores_bf16x3_kernel"}
        extra = {"scores_fp32_equiv_tflops": round(flop / score_avg_s / 1e12, 2),
                 "scores_frac_of_fp32_mfma_peak": round(flop / score_avg_s / 1e12 / PEAK_FP32_MFMA_TFLOPS, 4)}
    topk_bytes = 4.0 * (w.nq * w.active + w.nq * w.k)
    topk_avg_s = float(np.mean(topk_ms)) * 1e-3

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
        "dtype": "bf16x3" if path == "bf16x3" else "f32",
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
            "step_hbm_gbs": round(select_bytes / (ms_step * 1e-3) / 1e9, 1),
            "step_hbm_frac": round(select_bytes / (ms_step * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "scores_ms": round(float(np.mean(score_ms)), 5),
            "scores_ms_median": round(float(np.median(score_ms)), 5),
            "topk_ms": round(float(np.mean(topk_ms)), 5),
            "topk_ms_median": round(float(np.median(topk_ms)), 5),
            "topk_gbs": round(topk_bytes / topk_avg_s / 1e9, 1),
            "topk_hbm_frac": round(topk_bytes / topk_avg_s / 1e9 / PEAK_HBM_GBS, 4),
            "scores_kernel": path,
            **extra,
        },
        "roofline": roof,
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
        a_avg_s = float(np.mean(attn_ms)) * 1e-3
        gbs = abytes / a_avg_s / 1e9
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
        out["stages"]["attention_ms"] = round(float(np.mean(attn_ms)), 5)
        out["stages"]["attention_graph_replays_match_eager"] = attn_graph_ok
        out["roofline_attention"] = {
            "bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
            "bytes_per_call": int(abytes),
            "kernel": ("attn_chunk_i8_kernel" if int8 else "attn_chunk_kernel")
            + " + attn_merge_kernel (one call)"}
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, bt, args.cpu_threads, kv if attn else None)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
