#!/usr/bin/env python3
"""MoBA prefill forward on one MI355X: throughput, per-step times, roofline and the
CPU oracle baseline, printed as one JSON line.

    python bench.py [--steps K] [--warmup W] [--workload llama8b_128k] [--gpus 1]

A step is one whole moba_forward (centroid pool, gate + top-k, inverted index,
history attention, current-block attention fused with the merge) over one batch of
seeded synthetic inputs already resident in HBM.  `value` is effective TFLOP/s:
4 * head_dim * (keys each query head attends) summed over query heads and tokens,
divided by the step time.  The per-stage times (and so the roofline of the history
attention kernel) come from HIP events that the library records on the launch stream
at the stage boundaries of every timed step (moba_forward_timed, no synchronisation).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoBA prefill fwd ms + effective TFLOP/s at 128K, % bf16 MFMA peak (1 GPU)"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E, published
COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_history_llama8b_128k_counters.txt")
CURRENT_COUNTERS_FILE = os.path.join(ROOT, "profiles", "attn_current_llama8b_128k_counters.txt")
ATTN_SOURCE = os.path.join(ROOT, "block_sparse_long_pool_amd", "csrc", "attn.hip")


# ------------------------------------------------------------------ work counts
def pair_counts(T: int, B: int, k: int):
    """Per query head: (history pairs, current-block pairs) attended, from the
    definition: every row of block c attends min(c, k-1) whole blocks and the causal
    prefix of its own block (the last block may be partial)."""
    hist = cur = 0
    for c in range((T + B - 1) // B):
        n = min(B, T - c * B)
        hist += n * min(c, k - 1) * B
        cur += n * (n + 1) // 2
    return hist, cur


# packed-sequence mix timed beside the main workload: six requests of ragged lengths
# (131072 tokens in all), read out of the main workload's resident tensors
VARLEN_LENGTHS = (40000, 30000, 25000, 20000, 10000, 6072)
VARLEN_BLOCK, VARLEN_TOPK = 1024, 8


def gate_bytes(w, needed_only: bool) -> int:
    """Bytes of the gate step: every query row read once, the idx rows written, and the
    centroids (read as bf16 hi + lo, the size of fp32).  With needed_only, only the
    query rows that have more causal history blocks than slots are counted: the others
    select every causal block without a score, and the kernel never reads them."""
    nb = w.seqlen // w.block
    rows_per_block = w.batch * w.hq * w.block
    if needed_only:
        q_rows = rows_per_block * sum(1 for c in range(nb) if c > w.topk - 1)
    else:
        q_rows = rows_per_block * nb
    q = q_rows * w.head_dim * 2
    idx = w.batch * w.hq * w.seqlen * w.topk * 4
    cent = w.batch * w.hkv * nb * w.head_dim * 2 * 2
    return q + idx + cent


def source_hash(path: str) -> str:
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def history_kernel_name(w) -> str:
    """The history-attention kernel the library launches for this workload (the rule in
    launch_attn_history; the committed kernel statistics under profiles/ name the kernel
    that ran)."""
    if w.block <= 128:
        return "attn_history_resident_kernel (block resident in LDS, gathered query rows)"
    if w.block % 64 == 0 and 256 <= w.block <= 4096:
        return ("attn_history_chain_kernel (one persistent workgroup per CU, tiles from a "
                "queue, gathered query tiles)")
    return "attn_history_kernel (one workgroup per tile of gathered query rows)"


def read_counters(path: str, workload: str):
    """{'traffic': HBM bytes per dispatch, 'mfma_busy': fraction of SIMD cycles} from a
    committed rocprofv3 counter summary, or None when there is none, it was taken on
    another workload, or the kernel source changed since."""
    if not os.path.exists(path) or workload not in os.path.basename(path):
        return None
    text = open(path).read()
    m_h = re.search(r"source_sha256:\s*([0-9a-f]{64})", text)
    m_t = re.search(r"traffic_bytes_per_dispatch:\s*([0-9.eE+]+)", text)
    m_b = re.search(r"mfma_busy:\s*([0-9.eE+]+)", text)
    if not m_h or not m_t or m_h.group(1) != source_hash(ATTN_SOURCE):
        return None
    return {"traffic": float(m_t.group(1)),
            "mfma_busy": float(m_b.group(1)) if m_b else None,
            "file": os.path.relpath(path, ROOT)}


# ------------------------------------------------------------------ CPU oracle
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _cpu_worker(job):
    """One process of the CPU baseline: the oracle, as it is, on its query heads:
    full gating (centroids of its kv-heads, then the selection of every row of its
    heads), then attention of a stratified sample of its heads' rows until the
    deadline.  Inputs come from shared memory as bf16 bits."""
    import numpy as np
    from multiprocessing import shared_memory
    from threadpoolctl import threadpool_limits
    import oracle
    from workloads import bf16_to_f64

    (names, shapes, heads, G, B, k, scale, rows, t_attn) = job
    shm = [shared_memory.SharedMemory(name=n) for n in names]
    try:
        q, kk, vv = (np.ndarray(sh, np.uint16, buffer=m.buf) for sh, m in zip(shapes, shm))
        out = {"gate_s": 0.0, "attn_s": 0.0, "rows": 0, "pairs": 0}
        with threadpool_limits(limits=1):
            cache, qs = {}, {}
            t0 = time.perf_counter()
            for h in heads:
                g = h // G
                if g not in cache:
                    K = bf16_to_f64(kk[:, :, g:g + 1])
                    cache[g] = (K, bf16_to_f64(vv[:, :, g:g + 1]), oracle.centroids(K, B))
                qs[h] = bf16_to_f64(q[:, :, h:h + 1])
                oracle.select_blocks(qs[h], cache[g][2], B, k)
            out["gate_s"] = time.perf_counter() - t0
            t1 = time.perf_counter()
            T = q.shape[1]
            for (t, h) in rows:
                if time.perf_counter() - t1 > t_attn:
                    break
                K, V, C = cache[h // G]
                # the row's selection from its own gate scores, then one softmax over its
                # attended keys (the oracle's row functions, as the parity tests use them)
                _, _, sels, _ = oracle.moba_rows(qs[h], K, V, B, k, scale, [(0, t, 0)], C=C)
                out["pairs"] += oracle.attended_keys(sels[0], t, B, T).size
                out["rows"] += 1
            out["attn_s"] = time.perf_counter() - t1
        return out
    finally:
        for m in shm:
            m.close()


def cpu_baseline(w, inp, budget_s: float, workers: int):
    """The float64 oracle, as it is, over a process pool on the host's cores: full
    gating of every row, and attention on a stratified sample of rows (every query
    block, random token and head) for about ``budget_s`` seconds, extrapolated to the
    whole workload by attended (query, key) pairs."""
    import multiprocessing as mp
    from multiprocessing import shared_memory
    import numpy as np

    arrays = [inp["q"], inp["k"], inp["v"]]
    shm = []
    try:
        for a in arrays:
            m = shared_memory.SharedMemory(create=True, size=a.nbytes)
            np.ndarray(a.shape, np.uint16, buffer=m.buf)[...] = a
            shm.append(m)
        names = [m.name for m in shm]
        shapes = [a.shape for a in arrays]
        G = w.hq // w.hkv
        rng = np.random.default_rng(12345)
        nb = w.num_blocks
        # stratified sample, dealt to the workers by head
        sample = []
        for rep in range(max(64, 65536 // nb)):   # more rows than the deadline allows
            for c in range(nb):
                n = min(w.block, w.seqlen - c * w.block)
                sample.append((int(c * w.block + rng.integers(n)), int(rng.integers(w.hq))))
        jobs = []
        for i in range(workers):
            heads = list(range(i, w.hq, workers))
            rows = [r for r in sample if r[1] in heads]
            jobs.append((names, shapes, heads, G, w.block, w.topk, w.sm_scale, rows,
                         budget_s))
        jobs = [j for j in jobs if j[2]]
        ctx = mp.get_context("spawn")
        t0 = time.perf_counter()
        with ctx.Pool(len(jobs)) as pool:
            res = pool.map(_cpu_worker, jobs)
        wall = time.perf_counter() - t0
    finally:
        for m in shm:
            m.close()
            m.unlink()
    gate_wall = max(r["gate_s"] for r in res)
    attn_wall = max(r["attn_s"] for r in res)
    pairs = sum(r["pairs"] for r in res)
    rows = sum(r["rows"] for r in res)
    hist, cur = pair_counts(w.seqlen, w.block, w.topk)
    total_pairs = w.batch * w.hq * (hist + cur)
    total_flop = 4 * w.head_dim * total_pairs
    est_attn = attn_wall * total_pairs / max(pairs, 1)
    est_s = gate_wall + est_attn
    return {
        "value": total_flop / est_s / 1e12,
        "unit": "TFLOP/s",
        "cores": len(jobs),
        "kind": "oracle",
        "cpu_model": _cpu_model(),
        "host_cpus": len(os.sched_getaffinity(0)),
        "gating_s": gate_wall,
        "attention_s_extrapolated": est_attn,
        "sample": (f"{len(jobs)} processes, one BLAS thread each: full gating of all "
                   f"{w.batch * w.hq * w.seqlen} rows of {w.name} ({gate_wall:.1f} s), then "
                   f"attention of {rows} stratified sample rows (every query block, random "
                   f"token and head; {pairs} attended pairs) in {attn_wall:.1f} s, "
                   f"extrapolated by attended pairs to {est_attn:.0f} s; whole workload "
                   f"{est_s:.0f} s (pool wall {wall:.1f} s)"),
    }


# ------------------------------------------------------------------ achievable peaks
def achievable_peaks(dev):
    """A bf16 GEMM (torch.matmul, hipBLASLt) and a device copy, timed here, as the
    achievable MFMA and HBM rates next to the published peaks."""
    import torch
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    c = torch.empty(n, n, device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        torch.matmul(a, b, out=c)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    reps = 20
    for _ in range(reps):
        torch.matmul(a, b, out=c)
    e1.record()
    torch.cuda.synchronize()
    gemm_tflops = 2 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del a, b, c
    nbytes = 4 << 30
    src = torch.empty(nbytes // 2, device=dev, dtype=torch.bfloat16).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0.record()
    reps = 10
    for _ in range(reps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst
    return {
        "bf16_gemm_tflops": gemm_tflops,
        "bf16_gemm_frac_of_peak": gemm_tflops / PEAK_BF16_TFLOPS,
        "copy_gbs": copy_gbs,
        "copy_frac_of_peak": copy_gbs / PEAK_HBM_GBS,
        "note": f"torch.matmul {n}x{n}x{n} bf16 and a {nbytes >> 30} GiB device copy "
                "(read + write counted), timed in this run",
    }


# ------------------------------------------------------------------ one workload
def time_forward(moba, w, inp, dev, steps: int, warmup: int):
    """ms per whole forward and per stage on resident inputs (stage events recorded by
    the library on the launch stream in every timed step)."""
    import torch
    from workloads import to_torch_bf16
    q, k, v = (to_torch_bf16(inp[x], dev) for x in "qkv")
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.hq, w.seqlen), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.hq, w.seqlen, w.topk), dtype=torch.int32, device=dev)
    ws = moba.alloc_workspace(q, k, w.block, w.topk)
    for _ in range(warmup):
        moba.forward(q, k, v, w.block, w.topk, w.sm_scale, workspace=ws, out=out, lse=lse,
                     idx=idx)
    stream = torch.cuda.current_stream()
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(moba.STAGES) + 1)]
           for _ in range(steps)]
    for evs in sev:
        for e in evs:
            e.record(stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(steps):
        moba.forward(q, k, v, w.block, w.topk, w.sm_scale, workspace=ws, out=out, lse=lse,
                     idx=idx, events=sev[i])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    stage = {s_: sum(sev[i][j].elapsed_time(sev[i][j + 1]) for i in range(steps)) / steps
             for j, s_ in enumerate(moba.STAGES)}
    return ms, stage


def config_summary(w, ms, stage):
    hist, cur = pair_counts(w.seqlen, w.block, w.topk)
    flop = 4 * w.head_dim * w.batch * w.hq * (hist + cur)
    attn_ms = stage["history"] + stage["current"]
    gb = gate_bytes(w, needed_only=False)
    return {
        "ms": ms, "tflops": flop / (ms * 1e-3) / 1e12,
        "frac_of_bf16_peak": flop / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
        "attention_frac_of_bf16_peak": (flop / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
                                        if attn_ms > 0 else None),
        "gate_frac_of_hbm_peak": (gb / (stage["gate"] * 1e-3) / 1e9 / PEAK_HBM_GBS
                                  if stage["gate"] > 0 else None),
        "stages_ms": stage, "flop": flop,
        "shape": {"batch": w.batch, "seq_len": w.seqlen, "q_heads": w.hq, "kv_heads": w.hkv,
                  "head_dim": w.head_dim, "block": w.block, "topk": w.topk,
                  "recipe": w.recipe},
    }


# ------------------------------------------------------------------ main
def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="llama8b_128k")
    ap.add_argument("--cpu-seconds", type=float, default=20.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip timing dense causal attention on the same inputs")
    ap.add_argument("--no-graph", action="store_true",
                    help="skip timing the step captured in a HIP graph")
    ap.add_argument("--no-decode", action="store_true",
                    help="skip timing the full-attention decode step on the same cache")
    ap.add_argument("--no-conv", action="store_true",
                    help="skip timing the short key convolution")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip timing packed variable-length sequences")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing the backward pass (dQ, dK, dV) on the same inputs")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip timing the forward on the other workloads")
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the bf16 GEMM and device copy (achievable peaks)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes of the CPU oracle baseline (default: the host's CPUs, "
                         "at most 16)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="also run one elementwise copy (torch.neg) of this many MiB "
                         "of bf16, a kernel of known traffic for scaling HBM counters")
    a = ap.parse_args(argv)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if a.gpus != 1 or world != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {a.gpus}, WORLD_SIZE "
              f"{world}): the MoBA layer shards by kv-head with no communication, so "
              "the figure at N GPUs is N times the one-GPU figure on 1/N of the heads; "
              "this script measures one GPU.", file=sys.stderr)
        return 2

    import torch
    import block_sparse_long_pool_amd as moba
    from workloads import get_workload, make_inputs, to_torch_bf16

    w = get_workload(a.workload)
    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    inp = make_inputs(w)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    q = to_torch_bf16(inp["q"], dev)
    k = to_torch_bf16(inp["k"], dev)
    v = to_torch_bf16(inp["v"], dev)
    out = torch.empty_like(q)
    lse = torch.empty((w.batch, w.hq, w.seqlen), dtype=torch.float32, device=dev)
    idx = torch.empty((w.batch, w.hq, w.seqlen, w.topk), dtype=torch.int32, device=dev)
    ws = moba.alloc_workspace(q, k, w.block, w.topk)
    full_ws, _ = moba.workspace_bytes(w.batch, w.seqlen, w.hq, w.hkv, w.head_dim, w.block,
                                      w.topk)

    def step(events=None):
        return moba.forward(q, k, v, w.block, w.topk, w.sm_scale, workspace=ws, out=out,
                            lse=lse, idx=idx, events=events)

    print(f"[bench] warmup {a.warmup}", file=sys.stderr, flush=True)
    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # stage-boundary events for every timed step; one record each creates the HIP event
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(moba.STAGES) + 1)]
           for _ in range(a.steps)]
    for evs in sev:
        for e in evs:
            e.record(stream)
    print(f"[bench] timing {a.steps} steps", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(a.steps):
        step(events=sev[i])
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / a.steps

    graph_ms = None
    if not a.no_graph:
        # the same step captured once in a HIP graph and replayed: no per-kernel launch
        # cost (the library allocates, copies and clears nothing, so it captures as is)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step()
        g.replay()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(a.steps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_ms = e0.elapsed_time(e1) / a.steps
        del g

    if a.calibration_copy_mib:
        n = a.calibration_copy_mib * (1 << 20) // 2
        src = torch.ones(n, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.neg(src, out=dst)          # reads n*2 bytes, writes n*2 bytes
        torch.cuda.synchronize()
        print(f"[bench] calibration copy: {n * 2} bytes read, {n * 2} bytes written",
              file=sys.stderr, flush=True)
        del src, dst

    stage = {s_: sum(sev[i][j].elapsed_time(sev[i][j + 1]) for i in range(a.steps)) / a.steps
             for j, s_ in enumerate(moba.STAGES)}
    print(f"[bench] {ms:.3f} ms/step; stages {stage}", file=sys.stderr, flush=True)

    hist, cur = pair_counts(w.seqlen, w.block, w.topk)
    heads = w.batch * w.hq
    flop_hist = 4 * w.head_dim * heads * hist
    flop_cur = 4 * w.head_dim * heads * cur
    flop = flop_hist + flop_cur
    tflops = flop / (ms * 1e-3) / 1e12
    attn_ms = stage["history"] + stage["current"]
    hist_tflops = flop_hist / (stage["history"] * 1e-3) / 1e12 if stage["history"] else None
    gbytes = gate_bytes(w, needed_only=False)
    gbytes_needed = gate_bytes(w, needed_only=True)
    pbytes = w.batch * w.seqlen * w.hkv * w.head_dim * 2
    gate_s = stage["gate"] * 1e-3
    gate_gbs = gbytes / gate_s / 1e9 if gate_s else None
    gate_gbs_needed = gbytes_needed / gate_s / 1e9 if gate_s else None
    # history attention runs once per kv-head group; one launch covers all of them when
    # the workspace holds every head (it does for this workload)
    one_launch = ws.numel() >= full_ws
    hist_ctr = read_counters(COUNTERS_FILE, w.name) if one_launch else None
    cur_ctr = read_counters(CURRENT_COUNTERS_FILE, w.name) if one_launch else None
    roofline = {
        "bound": "mfma",
        "kernel": history_kernel_name(w),
        "achieved": hist_tflops,
        "peak": PEAK_BF16_TFLOPS,
        "unit": "TFLOP/s",
        "frac": hist_tflops / PEAK_BF16_TFLOPS if hist_tflops else None,
        "traffic": hist_ctr["traffic"] if hist_ctr else None,
        "mfma_busy": hist_ctr["mfma_busy"] if hist_ctr else None,
        "counters": hist_ctr["file"] if hist_ctr else None,
        "algorithmic_per_launch": f"{flop_hist:.4e} FLOP = 4 * d * {heads} heads * "
                                  f"{hist} history pairs per head",
    }
    result = {
        "metric": METRIC,
        "value": tflops,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "seq_len": w.seqlen,
                   "q_heads": w.hq, "kv_heads": w.hkv, "head_dim": w.head_dim,
                   "block": w.block, "topk": w.topk, "recipe": w.recipe},
        "frac_of_bf16_peak": tflops / PEAK_BF16_TFLOPS,
        "stages_ms": stage,
        "attention_tflops": flop / (attn_ms * 1e-3) / 1e12 if attn_ms else None,
        "attention_frac_of_bf16_peak": (flop / (attn_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
                                        if attn_ms else None),
        "gate_gbs": gate_gbs,
        "gate_frac_of_hbm_peak": gate_gbs / PEAK_HBM_GBS if gate_gbs else None,
        "gate_algorithmic_bytes": gbytes,
        "gate_needed_bytes": gbytes_needed,
        "gate_needed_gbs": gate_gbs_needed,
        "gate_needed_frac_of_hbm_peak": (gate_gbs_needed / PEAK_HBM_GBS
                                         if gate_gbs_needed else None),
        # the centroid pool reads every key once: T * Hkv * d bf16
        "pool_gbs": pbytes / (stage["pool"] * 1e-3) / 1e9 if stage["pool"] else None,
        "pool_frac_of_hbm_peak": (pbytes / (stage["pool"] * 1e-3) / 1e9 / PEAK_HBM_GBS
                                  if stage["pool"] else None),
        "pool_algorithmic_bytes": pbytes,
        "roofline": roofline,
        "current_kernel": {
            "ms": stage["current"],
            "tflops": flop_cur / (stage["current"] * 1e-3) / 1e12 if stage["current"] else None,
            "frac_of_bf16_peak": (flop_cur / (stage["current"] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS
                                  if stage["current"] else None),
            "traffic": cur_ctr["traffic"] if cur_ctr else None,
            "mfma_busy": cur_ctr["mfma_busy"] if cur_ctr else None,
            "note": "attn_current_kernel: causal current block fused with the merge of the "
                    "history partials",
        },
        "cpu_baseline": None,
    }
    if graph_ms is not None:
        result["graph_replay"] = {
            "ms_per_step": graph_ms, "tflops": flop / (graph_ms * 1e-3) / 1e12,
            "note": "the same step captured once in a HIP graph (torch.cuda.CUDAGraph) "
                    "and replayed: no per-launch cost",
        }
    if not a.no_dense:
        # the full-attention layer of a hybrid model on the same inputs: context for the
        # sparse path (not the metric)
        out_d = torch.empty_like(q)
        lse_d = torch.empty_like(lse)
        moba.dense_forward(q, k, v, w.sm_scale, out=out_d, lse=lse_d)
        n_dense = 3
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n_dense):
            moba.dense_forward(q, k, v, w.sm_scale, out=out_d, lse=lse_d)
        e1.record(stream)
        torch.cuda.synchronize()
        dms = e0.elapsed_time(e1) / n_dense
        dflop = 4 * w.head_dim * heads * w.seqlen * (w.seqlen + 1) // 2
        result["dense_causal"] = {
            "ms": dms, "tflops": dflop / (dms * 1e-3) / 1e12,
            "frac_of_bf16_peak": dflop / (dms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "moba_speedup": dms / ms,
            "note": "dense causal attention (moba_dense_forward) on the same inputs",
        }
        print(f"[bench] dense causal {dms:.2f} ms", file=sys.stderr, flush=True)
        del out_d, lse_d
    if not a.no_decode:
        # the hand-off after the prefill: one new token per sequence decoded with full
        # attention over the whole K/V cache (the last query row stands in for it).
        # HBM-bound: every cached key and value is read once.
        qd = q[:, -1:].contiguous()
        dws = torch.empty(max(moba.decode_workspace_bytes(w.batch, 1, w.seqlen, w.hq, w.hkv,
                                                          w.head_dim), 256),
                          dtype=torch.uint8, device=dev)
        od = torch.empty_like(qd)
        ld = torch.empty((w.batch, w.hq, 1), dtype=torch.float32, device=dev)

        def dstep():
            moba.decode(qd, k, v, w.sm_scale, workspace=dws, out=od, lse=ld)

        dstep()
        torch.cuda.synchronize()
        n_dec = 50
        e0.record(stream)
        for _ in range(n_dec):
            dstep()
        e1.record(stream)
        torch.cuda.synchronize()
        dec_ms = e0.elapsed_time(e1) / n_dec
        # algorithmic bytes: the cache's keys and values, the query and output rows
        dbytes = 2 * (2 * w.batch * w.seqlen * w.hkv * w.head_dim + 2 * w.batch * w.hq
                      * w.head_dim)
        result["decode"] = {
            "us": dec_ms * 1e3, "gbs": dbytes / (dec_ms * 1e-3) / 1e9,
            "frac_of_hbm_peak": dbytes / (dec_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "new_tokens": 1, "kv_len": w.seqlen, "algorithmic_bytes": dbytes,
            "note": "moba_decode: one new token against the 128K cache (full attention)",
        }
        print(f"[bench] decode {dec_ms * 1e3:.1f} us", file=sys.stderr, flush=True)
        del qd, dws, od, ld
    if not a.no_conv:
        # short key convolution within blocks (width 4, synthetic weights): HBM-bound,
        # every key read once and written once
        width = 4
        gw = torch.Generator(device=dev)
        gw.manual_seed(7)
        wconv = torch.randn(w.hkv, w.head_dim, width, device=dev, generator=gw) / 2.0
        kc = torch.empty_like(k)
        moba.key_short_conv(k, wconv, w.block, out=kc)
        torch.cuda.synchronize()
        n_conv = 20
        e0.record(stream)
        for _ in range(n_conv):
            moba.key_short_conv(k, wconv, w.block, out=kc)
        e1.record(stream)
        torch.cuda.synchronize()
        cms = e0.elapsed_time(e1) / n_conv
        # a plain device copy of the same bytes, for scale
        kc.copy_(k)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n_conv):
            kc.copy_(k)
        e1.record(stream)
        torch.cuda.synchronize()
        copy_ms = e0.elapsed_time(e1) / n_conv
        cbytes = 2 * k.numel() * 2
        result["key_short_conv"] = {
            "ms": cms, "gbs": cbytes / (cms * 1e-3) / 1e9,
            "frac_of_hbm_peak": cbytes / (cms * 1e-3) / 1e9 / PEAK_HBM_GBS,
            "width": width, "algorithmic_bytes": cbytes,
            "copy_gbs": cbytes / (copy_ms * 1e-3) / 1e9,
            "note": "moba_key_short_conv over the keys (read + write of k)",
        }
        print(f"[bench] key conv {cms:.3f} ms", file=sys.stderr, flush=True)
        del kc, wconv
    if not a.no_varlen and w.batch == 1 and w.seqlen == sum(VARLEN_LENGTHS):
        # packed variable-length prefill: the same tokens cut into six requests, each
        # with its own block grid (B = 1024, top-8, ragged last blocks)
        cu = [0]
        for n in VARLEN_LENGTHS:
            cu.append(cu[-1] + n)
        total = cu[-1]
        qv, kv, vv = (x.view(total, x.shape[2], x.shape[3]) for x in (q, k, v))
        full_v, _ = moba.varlen_workspace_bytes(len(VARLEN_LENGTHS), total,
                                                max(VARLEN_LENGTHS), w.hq, w.hkv, w.head_dim,
                                                VARLEN_BLOCK, VARLEN_TOPK)
        vws = torch.empty(full_v, dtype=torch.uint8, device=dev)
        vo = torch.empty_like(qv)
        vl = torch.empty((w.hq, total), dtype=torch.float32, device=dev)
        vi = torch.empty((w.hq, total, VARLEN_TOPK), dtype=torch.int32, device=dev)

        def vstep():
            moba.forward_varlen(qv, kv, vv, cu, VARLEN_BLOCK, VARLEN_TOPK, w.sm_scale,
                                workspace=vws, out=vo, lse=vl, idx=vi)

        vstep()
        torch.cuda.synchronize()
        n_var = 5
        e0.record(stream)
        for _ in range(n_var):
            vstep()
        e1.record(stream)
        torch.cuda.synchronize()
        vms = e0.elapsed_time(e1) / n_var
        vpairs = sum(sum(pair_counts(n, VARLEN_BLOCK, VARLEN_TOPK)) for n in VARLEN_LENGTHS)
        vflop = 4 * w.head_dim * w.hq * vpairs
        result["varlen"] = {
            "ms": vms, "tflops": vflop / (vms * 1e-3) / 1e12,
            "frac_of_bf16_peak": vflop / (vms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS,
            "lengths": list(VARLEN_LENGTHS), "block": VARLEN_BLOCK, "topk": VARLEN_TOPK,
            "flop": vflop,
            "note": "moba_forward_varlen: the main inputs' tokens as six packed requests",
        }
        print(f"[bench] varlen {vms:.2f} ms", file=sys.stderr, flush=True)
        if not a.no_backward:
            # the packed backward of the same requests (selection of the forward above)
            from workloads import make_output_grad
            vdout = to_torch_bf16(make_output_grad(w), dev).view(total, w.hq, w.head_dim)
            full_vb, _ = moba.backward_varlen_workspace_bytes(
                len(VARLEN_LENGTHS), total, max(VARLEN_LENGTHS), w.hq, w.hkv, w.head_dim,
                VARLEN_BLOCK, VARLEN_TOPK)
            vbws = torch.empty(full_vb, dtype=torch.uint8, device=dev)

            def vbstep():
                return moba.backward_varlen(qv, kv, vv, vo, vl, vi, vdout, cu, VARLEN_BLOCK,
                                            VARLEN_TOPK, w.sm_scale, workspace=vbws)

            vbstep()
            torch.cuda.synchronize()
            e0.record(stream)
            for _ in range(n_var):
                vbstep()
            e1.record(stream)
            torch.cuda.synchronize()
            vbms = e0.elapsed_time(e1) / n_var
            vbflop = 10 * w.head_dim * w.hq * vpairs
            result["varlen"].update({
                "backward_ms": vbms,
                "backward_effective_tflops": vbflop / (vbms * 1e-3) / 1e12,
                "backward_note": "moba_backward_varlen of the same requests, dout i.i.d. "
                                 "N(0,1); 10 d FLOP per attended pair",
            })
            print(f"[bench] varlen backward {vbms:.2f} ms", file=sys.stderr, flush=True)
            del vbws, vdout
        del vws, vo, vl, vi
    if not a.no_backward:
        # the training backward of the same layer (selection held fixed): context for
        # the forward metric.  FLOP conventions: "effective" counts the five products of
        # an attention backward (10 d per attended pair, 2.5x the forward's 4 d);
        # "executed" counts what the kernels run (14 d: S and dP are computed in both
        # the dQ and the dK/dV kernel).
        from workloads import make_output_grad
        dout = to_torch_bf16(make_output_grad(w), dev)
        full_b, min_b = moba.backward_workspace_bytes(w.batch, w.seqlen, w.hq, w.hkv,
                                                      w.head_dim, w.block, w.topk)
        bws = torch.empty(full_b, dtype=torch.uint8, device=dev)
        dq = torch.empty_like(q)
        dk = torch.empty_like(k)
        dv = torch.empty_like(v)

        def bstep():
            moba.backward(q, k, v, out, lse, idx, dout, w.block, w.topk, w.sm_scale,
                          workspace=bws, dq=dq, dk=dk, dv=dv)

        bstep()
        torch.cuda.synchronize()
        n_bwd = 3
        e0.record(stream)
        for _ in range(n_bwd):
            bstep()
        e1.record(stream)
        torch.cuda.synchronize()
        bms = e0.elapsed_time(e1) / n_bwd
        pairs = heads * (hist + cur)
        result["backward"] = {
            "ms": bms,
            "effective_tflops": 10 * w.head_dim * pairs / (bms * 1e-3) / 1e12,
            "effective_frac_of_bf16_peak": (10 * w.head_dim * pairs / (bms * 1e-3) / 1e12
                                            / PEAK_BF16_TFLOPS),
            "executed_tflops": 14 * w.head_dim * pairs / (bms * 1e-3) / 1e12,
            "forward_plus_backward_ms": ms + bms,
            "workspace_bytes": full_b,
            "note": "moba_backward (dq, dk, dv) on the same inputs, dout i.i.d. N(0,1)",
        }
        print(f"[bench] backward {bms:.2f} ms", file=sys.stderr, flush=True)
        del bws, dq, dk, dv, dout
    if not a.no_configs:
        # the forward on the other workloads of the benchmark plan (one GPU each); the
        # headline line above stays the 128K one
        del q, k, v, out, lse, idx, ws
        torch.cuda.empty_cache()
        result["configs"] = {}
        for name in ("tiny_2k", "llama8b_32k", "llama8b_64k_b128"):
            if name == w.name:
                continue
            wc = get_workload(name)
            print(f"[bench] {name}: generating inputs", file=sys.stderr, flush=True)
            ic = make_inputs(wc)
            cms, cstage = time_forward(moba, wc, ic, dev, steps=max(a.steps, 10), warmup=3)
            result["configs"][name] = config_summary(wc, cms, cstage)
            print(f"[bench] {name}: {cms:.3f} ms; stages {cstage}", file=sys.stderr,
                  flush=True)
            del ic
            torch.cuda.empty_cache()
    if not a.no_peaks:
        result["achievable_peaks"] = achievable_peaks(dev)
        print(f"[bench] peaks {result['achievable_peaks']}", file=sys.stderr, flush=True)
    if not a.no_cpu_baseline:
        workers = a.cpu_workers or min(16, len(os.sched_getaffinity(0)))
        print(f"[bench] CPU oracle baseline ({workers} processes, ~{a.cpu_seconds:.0f} s of "
              "attention)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, inp, a.cpu_seconds, workers)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
