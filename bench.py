#!/usr/bin/env python3
"""Benchmark of the DSA decode hot path on one MI355X.

A step is one dsa_forward call (lightning indexer -> top-2048 -> sparse
absorbed MLA) over one batch of synthetic inputs already resident in HBM.
The headline workload is batch-1 decode at 32768 cached tokens in bf16
(64x128 indexer, 128-head 512+64 MLA).  Inputs are rotated over enough
copies (>= 1 GiB in total) that every step reads its caches from HBM rather
than from the 256 MB last-level cache.

Printed: one JSON line with the throughput (query tokens/s; the mean over
exactly --steps steps, plus the median/p10/p90 of 50 further graph replays),
each stage's achieved rate against its roof (HBM bytes against 8 TB/s and
against a measured device copy, MFMA FLOPs against the bf16 peak for the
prefill), a roofline entry for the dominant stage (algorithmic bytes per call
/ average call time, from HIP events on the launch stream), the same figures
for the batch-64 fp8 decode and the 8192-query prefill workloads, the CPU
oracle timed on a bounded sample of each workload, the measured
sparse-vs-dense break-even context of the batch-8 fp8 sweep, and the headline
step through the library's captured-step API (one graph launch per step).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, GB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA
METRIC = "sparse-attn decode query-tok/s at 32K ctx; % HBM roofline; dense break-even"
ROTATION_BYTES = 1 << 30

# Algorithmic work.  The step figures count the compulsory traffic of the
# method's inputs and output (intermediates excluded); the per-stage figures
# add each stage's own intermediate I/O (scores written by the indexer and
# read by the selection, indices written and read).
def indexer_bytes(n_keys_total, rows, fp8):
    per_key = 132 if fp8 else 256            # 128-dim key (+ fp32 scale for fp8)
    per_row = (8192 + 256 + 256) if fp8 else (16384 + 256)  # q (+ q_scale) + weights
    return per_key * n_keys_total + per_row * rows


def sparse_mla_bytes(n_selected_total, rows):
    # gathered 512+64 bf16 rows, q_nope+q_pe (147456 B), bf16 output (131072 B)
    return 1152 * n_selected_total + (147456 + 131072) * rows


def dense_mla_bytes(n_keys_total, rows):
    return 1152 * n_keys_total + (147456 + 131072) * rows


def topk_bytes(n_scores_total, rows, k):
    return 4 * n_scores_total + 4 * k * rows


def stage_work(case):
    """Per-stage algorithmic work of one dsa_forward call on `case`: HBM bytes for
    every stage, plus MFMA FLOPs for the indexer and attention of a prefill."""
    ep = [int(x) for x in case.end_pos.cpu().tolist()]
    B, T, k = case.B, case.T, case.topk
    fp8 = case.dtype == "fp8"
    bounds = [e - T + t + 1 for e in ep for t in range(T)]     # valid keys per query row
    sel = sum(min(k, n) for n in bounds)
    pairs = sum(bounds)
    keys = sum(ep)                                              # each cached key read once
    rows = B * T
    w = {
        "index_scores": {"bytes": indexer_bytes(keys, rows, fp8) + 4 * pairs,
                         "flop": 2 * 64 * 128 * pairs},
        "topk": {"bytes": topk_bytes(pairs, rows, k)},
        "sparse_mla": {"bytes": sparse_mla_bytes(sel, rows) + (512 + 4 * k) * rows,
                       "flop": 2 * 128 * (576 + 512) * sel},
    }
    step = indexer_bytes(keys, rows, fp8) + sparse_mla_bytes(sel, rows)
    return w, step


# The HIP kernels behind each stage of the batch-1 32K decode step (a
# stage's time is the sum of its kernels' launch durations plus the gaps
# between them).
STAGE_KERNELS = {
    "index_scores": ["indexer_kernel<false>"],
    "topk": ["topk_cut_kernel<4>", "topk_pick_kernel<4>"],
    "sparse_mla": ["mla_tile_kernel<false>", "mla_combine_kernel<32, 4>"],
}


def source_digest(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sparse_attention_indexer_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel_file, digest):
    """HBM bytes per launch from a committed PMC summary, if it was taken on this source."""
    path = os.path.join(ROOT, "profiles", kernel_file)
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != digest:
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


class Timer:
    """Times calls of fn(i) with HIP events on the stream they run on.

    `reps` calls are captured into one HIP graph (torch.cuda.CUDAGraph) and
    replayed on the current stream, once untimed, then between two events
    recorded on that same stream, so the timed region holds exactly `reps`
    calls and measures the GPU, not the Python launch loop.
    """

    def __init__(self, torch):
        self.torch = torch

    def _graph(self, fn, reps):
        t = self.torch
        g = t.cuda.CUDAGraph()
        stream = t.cuda.Stream()
        stream.wait_stream(t.cuda.current_stream())
        with t.cuda.stream(stream):
            with t.cuda.graph(g, stream=stream):
                for i in range(reps):
                    fn(i)
        t.cuda.current_stream().wait_stream(stream)
        g.replay()  # warm replay
        t.cuda.synchronize()
        return g

    def time(self, fn, reps):
        """Mean ms per call over one replay of a graph of `reps` calls."""
        t = self.torch
        g = self._graph(fn, reps)
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        t.cuda.synchronize()
        s.record()
        g.replay()
        e.record()
        t.cuda.synchronize()
        return s.elapsed_time(e) / reps

    def dist(self, fn, per_graph, replays=50):
        """ms per call of each of `replays` timed replays of a graph of `per_graph` calls."""
        t = self.torch
        g = self._graph(fn, per_graph)
        ev = [(t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True))
              for _ in range(replays)]
        t.cuda.synchronize()
        for s, e in ev:
            s.record()
            g.replay()
            e.record()
        t.cuda.synchronize()
        return [s.elapsed_time(e) / per_graph for s, e in ev]


def percentiles(xs):
    ys = sorted(xs)

    def q(p):
        i = p * (len(ys) - 1)
        lo = int(math.floor(i))
        hi = min(lo + 1, len(ys) - 1)
        return ys[lo] + (ys[hi] - ys[lo]) * (i - lo)
    return {"median_ms": round(q(0.5), 5), "p10_ms": round(q(0.1), 5), "p90_ms": round(q(0.9), 5),
            "replays": len(ys)}


def case_bytes(case):
    tot = 0
    for name in ("q", "w", "k_cache", "q_scale", "k_scale", "q_nope", "q_pe", "kv_cache",
                 "pe_cache"):
        v = getattr(case, name)
        if v is not None:
            tot += v.numel() * v.element_size()
    return tot


def clone_case(case):
    from dataclasses import fields
    from sparse_attention_indexer_amd.inputs import Case
    kw = {}
    for f in fields(case):
        v = getattr(case, f.name)
        kw[f.name] = v.clone() if hasattr(v, "clone") else v
    return Case(**kw)


def rotation(case, limit=64):
    n = max(1, min(limit, math.ceil(ROTATION_BYTES / max(1, case_bytes(case)))))
    return [case] + [clone_case(case) for _ in range(n - 1)]


def bench_workload(dsa, torch, case, steps, warmup, per_kernel=True, replays=50):
    """Time dsa_forward over rotated input copies: the mean over exactly `steps`
    steps, the distribution over `replays` further replays, and (per_kernel)
    each stage's C-ABI call on its own."""
    copies = rotation(case)
    B, T, S, k = case.B, case.T, case.S_max, case.topk
    dev = case.q.device
    mep = case.max_end_pos
    ws = torch.zeros(dsa.forward_workspace_size(B, T, S, k), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T, 128), dtype=torch.float32, device=dev)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)

    def step(i):
        c = copies[i % len(copies)]
        dsa.forward(c.q, c.w, c.k_cache, c.end_pos, c.q_nope, c.q_pe, c.kv_cache, c.pe_cache,
                    c.scale, c.softmax_scale, k=k, q_scale=c.q_scale, k_scale=c.k_scale,
                    max_end_pos=mep, out=out, lse=lse, topk_out=idx, workspace=ws)

    timer = Timer(torch)
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    ms = timer.time(step, steps)
    res = {"ms_per_step": ms, "copies": len(copies)}
    if replays:
        per_graph = max(1, min(20, int(0.5 / max(ms, 1e-4))))  # about 0.5 ms per replay
        res.update(percentiles(timer.dist(step, per_graph, replays)))
        res["steps_per_replay"] = per_graph
    if not per_kernel:
        return res

    scores = torch.empty((B, T, S), dtype=torch.float32, device=dev)

    def st_index(i):
        c = copies[i % len(copies)]
        dsa.index_scores(c.q, c.w, c.k_cache, c.end_pos, c.scale, q_scale=c.q_scale,
                         k_scale=c.k_scale, max_end_pos=mep, out=scores)

    topk_ws = torch.zeros(max(1, dsa.lib().dsa_topk_workspace_size(B, T, S, k)),
                          dtype=torch.uint8, device=dev)

    def st_topk(i):
        dsa.topk(scores, copies[i % len(copies)].end_pos, k, max_end_pos=mep, out=idx,
                 workspace=topk_ws)

    mla_ws = torch.empty(max(1, dsa.lib().dsa_sparse_mla_workspace_size(B, T, k)),
                         dtype=torch.uint8, device=dev)

    def st_mla(i):
        c = copies[i % len(copies)]
        dsa.sparse_mla(c.q_nope, c.q_pe, c.kv_cache, c.pe_cache, idx, c.softmax_scale, out=out,
                       lse=lse, workspace=mla_ws)

    reps = max(5, min(200, int(20.0 / max(ms, 1e-4))))  # about 20 ms of work per stage
    for fn in (st_index, st_topk, st_mla):
        fn(0)
    res["stage_ms"] = {"index_scores": timer.time(st_index, reps),
                       "topk": timer.time(st_topk, reps),
                       "sparse_mla": timer.time(st_mla, reps)}
    res["stage_reps"] = reps
    del scores, topk_ws, mla_ws
    return res


def bench_library_graph(dsa, torch, case, steps, warmup):
    """The step through the library's own captured decode step: one
    dsa_forward_graph_create per rotated input copy, then exactly `steps`
    dsa_forward_graph_launch calls (one per step, round robin over the copies)
    between two events on the launch stream."""
    copies = rotation(case)
    B, T, S, k = case.B, case.T, case.S_max, case.topk
    dev = case.q.device
    ws = torch.zeros(dsa.forward_workspace_size(B, T, S, k), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T, 128), dtype=torch.float32, device=dev)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    graphs = [dsa.ForwardGraph(c.q, c.w, c.k_cache, c.end_pos, c.q_nope, c.q_pe, c.kv_cache,
                               c.pe_cache, c.scale, c.softmax_scale, out, lse, idx, ws, k=k,
                               q_scale=c.q_scale, k_scale=c.k_scale, max_end_pos=c.max_end_pos)
              for c in copies]
    stream = torch.cuda.current_stream()
    for i in range(max(warmup, len(graphs))):
        graphs[i % len(graphs)].launch(stream)
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record(stream)
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].launch(stream)
    host_us = (time.perf_counter() - t0) / steps * 1e6
    e.record(stream)
    torch.cuda.synchronize()
    ms = s.elapsed_time(e) / steps
    for g in graphs:
        g.close()
    # For comparison: the same steps as plain dsa_forward calls (five kernel launches
    # each, no graph).
    def eager(i):
        c = copies[i % len(copies)]
        dsa.forward(c.q, c.w, c.k_cache, c.end_pos, c.q_nope, c.q_pe, c.kv_cache, c.pe_cache,
                    c.scale, c.softmax_scale, k=k, q_scale=c.q_scale, k_scale=c.k_scale,
                    max_end_pos=c.max_end_pos, out=out, lse=lse, topk_out=idx, workspace=ws,
                    stream=stream)
    for i in range(warmup):
        eager(i)
    torch.cuda.synchronize()
    s.record(stream)
    t0 = time.perf_counter()
    for i in range(steps):
        eager(i)
    eager_host_us = (time.perf_counter() - t0) / steps * 1e6
    e.record(stream)
    torch.cuda.synchronize()
    eager_ms = s.elapsed_time(e) / steps
    return {"ms_per_step": round(ms, 5), "query_tok_s": round(B * T / (ms * 1e-3), 1),
            "graphs": len(graphs), "steps": steps, "host_us_per_launch": round(host_us, 2),
            "eager_ms_per_step": round(eager_ms, 5), "eager_host_us_per_step": round(eager_host_us, 2)}


def stage_fractions(stage_ms, work, copy_gbs, mfma_stages=()):
    """Per-stage achieved rate against its roof: HBM bytes / time against 8 TB/s and
    against the measured copy bandwidth, or (mfma_stages) FLOPs / time against
    the bf16 MFMA peak."""
    out = {}
    for name, t in stage_ms.items():
        w = work[name]
        gbs = w["bytes"] / (t * 1e-3) / 1e9
        e = {"ms": round(t, 5), "bytes": w["bytes"], "achieved_gbs": round(gbs, 1),
             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        if copy_gbs:
            e["hbm_frac_vs_copy"] = round(gbs / copy_gbs, 4)
        if name in mfma_stages:
            tf = w["flop"] / (t * 1e-3) / 1e12
            e.update({"flop": w["flop"], "achieved_tflops": round(tf, 1),
                      "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
        out[name] = e
    return out


def copy_bandwidth(torch, dev, nbytes=1 << 30, reps=20):
    """Device-to-device copy of `nbytes` (read + write counted): measured GB/s."""
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    ms = Timer(torch).time(lambda i: dst.copy_(src), reps)
    del src, dst
    torch.cuda.empty_cache()
    return {"bytes_per_copy": 2 * nbytes, "ms": round(ms, 4),
            "gbs": round(2 * nbytes / (ms * 1e-3) / 1e9, 1)}


def rocminfo_peaks():
    """Compute units and maximum engine clock of the first gfx950 agent, and the
    dense bf16/fp8 MFMA peaks they give (4096 and 8192 FLOP per clock per CU)."""
    import subprocess
    try:
        txt = subprocess.run(["rocminfo"], capture_output=True, text=True, timeout=60).stdout
    except (OSError, subprocess.SubprocessError):
        return None
    cus = clk = None
    for block in txt.split("*******")[1:]:
        if "gfx950" not in block:
            continue
        for line in block.splitlines():
            if line.strip().startswith("Compute Unit:"):
                cus = int(line.split(":")[1])
            elif line.strip().startswith("Max Clock Freq. (MHz):"):
                clk = int(line.split(":")[1])
        if cus and clk:
            break
    if not (cus and clk):
        return None
    return {"compute_units": cus, "max_sclk_mhz": clk,
            "bf16_dense_tflops": round(cus * clk * 1e6 * 4096 / 1e12, 1),
            "fp8_dense_tflops": round(cus * clk * 1e6 * 8192 / 1e12, 1),
            "hbm_gbs_spec": HBM_PEAK_GBS}


def bench_dense(dsa, torch, case, steps, warmup):
    copies = rotation(case)
    B, T, S = case.B, case.T, case.S_max
    dev = case.q.device
    mep = case.max_end_pos
    ws = torch.empty(max(1, dsa.lib().dsa_dense_mla_workspace_size(B, T, S)), dtype=torch.uint8,
                     device=dev)
    out = torch.empty((B, T, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T, 128), dtype=torch.float32, device=dev)

    def step(i):
        c = copies[i % len(copies)]
        dsa.dense_mla(c.q_nope, c.q_pe, c.kv_cache, c.pe_cache, c.end_pos, c.softmax_scale,
                      max_end_pos=mep, out=out, lse=lse, workspace=ws)

    for i in range(warmup):
        step(i)
    return Timer(torch).time(step, steps)


def bench_projections(dsa, torch, B, T, steps, dev):
    """Query absorption and output up-projection at B x T query rows: time per
    call and the HBM roofline of their 16.8 MB per-call weight stream."""
    from sparse_attention_indexer_amd import inputs
    qn, wkv, x = inputs.make_proj(B, T, seed=1, device=dev)
    n = max(1, min(64, math.ceil(ROTATION_BYTES / (wkv.numel() * 2))))
    w = [wkv] + [wkv.clone() for _ in range(n - 1)]  # rotate the weights through HBM
    qa = torch.empty((B, T, 128, 512), dtype=torch.bfloat16, device=dev)
    y = torch.empty((B, T, 128, 128), dtype=torch.bfloat16, device=dev)
    timer = Timer(torch)
    res = {}
    R = B * T
    for name, fn, act in (("q_absorb", lambda i: dsa.q_absorb(qn, w[i % n], out=qa), 128 + 512),
                          ("out_proj", lambda i: dsa.out_proj(x, w[i % n], out=y), 512 + 128)):
        fn(0)
        ms = timer.time(fn, steps)
        nbytes = 128 * 128 * 512 * 2 + R * 128 * act * 2
        gbs = nbytes / (ms * 1e-3) / 1e9
        res[name] = {"rows": R, "us": round(ms * 1e3, 2), "bytes": nbytes,
                     "achieved_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
    return res


def prep_bytes(tokens, fp8=True):
    """Algorithmic HBM bytes of the indexer input preparation for `tokens` new
    tokens: per token 64 query heads + 1 key of 128 bf16 in, one 128-byte cos and
    sin table row in, and 65 rotated vectors out (fp8 codes + one fp32 scale
    each, or bf16)."""
    out = 65 * (128 + 4) if fp8 else 65 * 256
    return tokens * (65 * 256 + 2 * 128 + out)


def bench_prep(dsa, torch, steps, dev, shapes=((1, 1), (64, 1), (1, 8192))):
    """Indexer input preparation (fp8 cache) at decode batch 1, decode batch 64
    and one 8192-token prefill chunk: time per call and its HBM roofline."""
    from sparse_attention_indexer_amd import inputs
    timer = Timer(torch)
    res = {}
    for B, T in shapes:
        S_max = max(T, 4096)
        per = prep_bytes(B * T)
        n = max(2, min(16, math.ceil(ROTATION_BYTES / 2 / per)))   # copies rotated through HBM
        sets = []
        for i in range(n):
            q_in, k_in, cos, sin, ep = inputs.make_prep(B, T, [S_max] * B, S_max, seed=90 + i,
                                                        device=dev)
            kc = torch.zeros((B, S_max, 128), dtype=torch.float8_e4m3fn, device=dev)
            ks = torch.zeros((B, S_max), dtype=torch.float32, device=dev)
            qo = torch.empty((B, T, 64, 128), dtype=torch.float8_e4m3fn, device=dev)
            qs = torch.empty((B, T, 64), dtype=torch.float32, device=dev)
            sets.append((q_in, k_in, cos, sin, ep, kc, ks, qo, qs))

        def fn(i):
            q_in, k_in, cos, sin, ep, kc, ks, qo, qs = sets[i % n]
            dsa.indexer_prep(q_in, k_in, cos, sin, ep, kc, ks, q_out=qo, q_scale=qs)
        fn(0)
        ms = timer.time(fn, steps)
        gbs = per / (ms * 1e-3) / 1e9
        res[f"b{B}_t{T}"] = {"tokens": B * T, "us": round(ms * 1e3, 2), "bytes": per,
                             "achieved_gbs": round(gbs, 1),
                             "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}
        del sets
        torch.cuda.empty_cache()
    return res


def bench_mha_prefill(dsa, torch, steps, dev, T=8192, k=2048):
    """MHA-form prefill attention on one T-token sequence with k random causal
    selections per query: time per call and MFMA roofline of the algorithmic
    FLOPs (selected (query, key) pairs x 128 heads x (192 + 128) x 2)."""
    from sparse_attention_indexer_amd import inputs
    q, kn, kp, v = inputs.make_mha(1, T, seed=7, device=dev)
    idx = inputs.make_indices(1, T, [T], k, seed=7, fill="random", device=dev)
    out = torch.empty((1, T, 128, 128), dtype=torch.bfloat16, device=dev)
    ws = torch.zeros(int(dsa.lib().dsa_sparse_mha_prefill_workspace_size(1, T)), dtype=torch.uint8,
                     device=dev)
    fn = lambda i: dsa.sparse_mha_prefill(q, kn, kp, v, idx, 192 ** -0.5, out=out,
                                          want_lse=False, workspace=ws)
    fn(0)
    ms = Timer(torch).time(fn, steps)
    pairs = sum(min(k, s + 1) for s in range(T))
    flop = pairs * 128 * (192 + 128) * 2
    tf = flop / (ms * 1e-3) / 1e12
    return {"workload": f"prefill_{T}_mha_bf16", "ms": round(ms, 4), "pairs": pairs,
            "algorithmic_flop": flop, "achieved_tflops": round(tf, 1),
            "mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}


def break_even(contexts, sparse_ms, dense_ms):
    """Context where sparse and dense times cross (log-linear interpolation), or None."""
    diff = [s - d for s, d in zip(sparse_ms, dense_ms)]
    for i in range(1, len(contexts)):
        if diff[i - 1] > 0 >= diff[i]:
            x0, x1 = math.log(contexts[i - 1]), math.log(contexts[i])
            f = diff[i - 1] / (diff[i - 1] - diff[i])
            return round(math.exp(x0 + f * (x1 - x0)))
    if diff and diff[0] <= 0:
        return contexts[0]
    return None


_CASE_ARRAYS = ("q", "w", "k_cache", "q_scale", "k_scale", "end_pos", "q_nope", "q_pe",
                "kv_cache", "pe_cache")


def _host(case, b0=None, b1=None):
    """Host copies of the case's arrays (sequences b0:b1 only, if given)."""
    from sparse_attention_indexer_amd import inputs
    h = {}
    for n in _CASE_ARRAYS:
        v = getattr(case, n)
        if v is not None and b0 is not None:
            v = v[b0:b1]
        h[n] = None if v is None else inputs.to_numpy(v)
    return h


def _oracle_step(h, case, rows=None):
    import numpy as np

    import oracle
    s = oracle.index_scores(h["q"], h["w"], h["k_cache"], h["end_pos"], case.scale,
                            q_scale=h["q_scale"], k_scale=h["k_scale"], rows=rows)
    idx = oracle.topk(np.nan_to_num(s, nan=0.0), h["end_pos"], case.topk, rows=rows)
    oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"], h["end_pos"],
               case.softmax_scale, indices=idx, rows=rows)


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), for the CPU baselines."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(case, budget_s=15.0):
    """The CPU oracle (as it stands) on a bounded sample: whole decode steps of the workload."""
    import oracle
    h = _host(case)
    reps, t0 = 0, time.perf_counter()
    while True:
        _oracle_step(h, case)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 2000:
            break
    q_tok = reps * case.B * case.T
    return {"value": q_tok / el, "unit": "query-tok/s", "cores": oracle.max_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{reps} whole decode step(s) of {case.name} (B={case.B}, T={case.T}, "
                      f"n={case.max_end_pos}): fp64 indexer over every key, full-sort top-"
                      f"{case.topk}, masked-softmax MLA over 128 heads; {el:.1f} s"}


def cpu_baseline_decode_sample(case, budget_s=10.0):
    """The oracle on whole sequences of a decode batch, one at a time in a fixed
    order, until the budget is spent: query-tok/s over that sample (each
    sequence is one query at its own context length)."""
    import oracle
    order = [int(x) for x in case.end_pos.argsort().tolist()]
    order = order[len(order) // 2:] + order[:len(order) // 2]  # from the median length up
    done, keys, t0 = 0, 0, time.perf_counter()
    for b in order:
        h = _host(case, b, b + 1)
        _oracle_step(h, case)
        done += 1
        keys += int(h["end_pos"][0])
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "query-tok/s", "cores": oracle.max_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{done} of the {case.B} sequences of {case.name} (mean context "
                      f"{keys // max(1, done)}), each a whole decode step; {el:.1f} s"}


def cpu_baseline_prefill_sample(case, budget_s=10.0, n_rows=1024):
    """The oracle on a sample of the query rows of a prefill (scores over the
    row's causal prefix, its top-k, its attention), until the budget is spent:
    query-tok/s over that sample.  The rows are n_rows evenly spaced ones, in
    an order that keeps any prefix of the sample spread over the sequence."""
    rows = sorted(range(n_rows), key=lambda i: int(f"{i:010b}"[::-1], 2))  # bit-reversed
    rows = [case.T - 1 - (i * case.T) // n_rows for i in rows]
    import numpy as np

    import oracle
    from sparse_attention_indexer_amd import inputs
    done, t0 = 0, time.perf_counter()
    for r in rows:
        # Query row r sees keys 0..start+r: the same work as a one-query decode
        # step over that prefix.
        n = int(case.end_pos[0]) - case.T + r + 1
        h = {}
        for name in _CASE_ARRAYS:
            v = getattr(case, name)
            if v is None or name == "end_pos":
                h[name] = None
            elif name in ("k_cache", "kv_cache", "pe_cache", "k_scale"):
                h[name] = inputs.to_numpy(v[:1, :n])
            else:
                h[name] = inputs.to_numpy(v[:1, r:r + 1])
        h["end_pos"] = np.array([n], dtype=np.int32)
        _oracle_step(h, case)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": done / el, "unit": "query-tok/s", "cores": oracle.max_threads(), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{done} of {n_rows} evenly spaced query rows of {case.name} "
                      f"(T={case.T}), each scored, selected and attended on its own; "
                      f"{el:.1f} s"}


def bench_leg(dsa, torch, case, steps, warmup, copy_gbs, mfma_stages=(), replays=50):
    """One further workload: step time and distribution, throughput and the
    per-stage fractions."""
    r = bench_workload(dsa, torch, case, steps, warmup, replays=replays)
    work, step_bytes = stage_work(case)
    ms = r["ms_per_step"]
    leg = {"workload": case.name, "batch": case.B, "queries_per_seq": case.T,
           "max_context": case.max_end_pos, "ms_per_step": round(ms, 5),
           "query_tok_s": round(case.B * case.T / (ms * 1e-3), 1),
           **{k: r[k] for k in ("median_ms", "p10_ms", "p90_ms", "replays", "steps_per_replay")},
           "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
           "stages": stage_fractions(r["stage_ms"], work, copy_gbs, mfma_stages),
           "stage_reps": r["stage_reps"], "input_copies": r["copies"]}
    return leg


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true", help="skip the sparse-vs-dense sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baselines")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the batch-64 fp8 decode and 8192-query prefill workloads")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the projections, indexer input preparation and MHA prefill")
    ap.add_argument("--only", choices=("decode_32k", "decode_b64", "prefill_8192"), default=None,
                    help="time only this workload's dsa_forward steps (for profiler runs)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--detail", default=None, help="also write per-config details (JSON) here")
    args = ap.parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the path has no "
              "multi-GPU mode.", file=sys.stderr)
        return 2

    import torch

    import sparse_attention_indexer_amd as dsa
    from sparse_attention_indexer_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    dsa.lib()  # fail loudly if the HIP library is missing
    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")

    if args.only:
        make = {"decode_32k": lambda: inputs.decode_32k(device=dev),
                "decode_b64": lambda: inputs.decode_b64_varlen(device=dev),
                "prefill_8192": lambda: inputs.prefill(8192, device=dev)}[args.only]
        case = make()
        r = bench_workload(dsa, torch, case, args.steps, args.warmup, per_kernel=False, replays=0)
        print(json.dumps({"workload": case.name, "steps": args.steps,
                          "ms_per_step": round(r["ms_per_step"], 5)}), flush=True)
        return 0

    copy = copy_bandwidth(torch, dev)
    copy_gbs = copy["gbs"]

    # --- headline: batch-1 decode at 32K, bf16 ---
    case = inputs.decode_32k(device=dev)
    r = bench_workload(dsa, torch, case, args.steps, args.warmup)
    B, T, n, k = case.B, case.T, case.max_end_pos, case.topk
    ms = r["ms_per_step"]
    value = B * T / (ms * 1e-3)
    work, step_bytes = stage_work(case)
    st = r["stage_ms"]
    stages = stage_fractions(st, work, copy_gbs)
    dom = max(st, key=st.get)
    achieved = work[dom]["bytes"] / (st[dom] * 1e-3) / 1e9
    digest_files = {"index_scores": ["indexer.hip"], "topk": ["topk.hip", "select.h"],
                    "sparse_mla": ["mla.hip"]}[dom]
    traffic = read_traffic(f"{dom}_decode_32k_bf16.pmc.txt", source_digest(digest_files))
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tok/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode_32k_bf16", "batch": B, "queries_per_seq": T,
                   "context": n, "topk": k, "index_heads": 64, "index_dim": 128,
                   "mla_heads": 128, "latent": 512, "rope": 64, "input_copies": r["copies"]},
        "roofline": {"bound": "hbm", "kernel": dom, "kernels": STAGE_KERNELS[dom],
                     "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "algorithmic_bytes_per_launch": work[dom]["bytes"],
                     "avg_launch_ms": round(st[dom], 5),
                     "frac_vs_copy": round(achieved / copy_gbs, 4)},
        "step": {k2: r[k2] for k2 in ("median_ms", "p10_ms", "p90_ms", "replays",
                                       "steps_per_replay")},
        "stages": stages,
        "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_algorithmic_bytes": step_bytes,
        "copy_bandwidth": copy,
        "peaks": rocminfo_peaks(),
    }
    # The same step through the library's captured-step API (one launch call a step).
    line["library_graph_step"] = bench_library_graph(dsa, torch, case, args.steps, args.warmup)
    detail = {"headline": r}
    host_case = case.to("cpu")
    del case
    torch.cuda.empty_cache()

    legs = {}
    if not args.no_legs:
        # Batch-64 decode, contexts uniform in [8192, 131072], fp8 indexer.
        c3 = inputs.decode_b64_varlen(device=dev)
        legs["decode_b64_varlen_fp8"] = bench_leg(dsa, torch, c3, max(20, args.steps // 4), 5,
                                                  copy_gbs)
        if not args.no_cpu:
            legs["decode_b64_varlen_fp8"]["cpu_baseline"] = cpu_baseline_decode_sample(c3)
        del c3
        torch.cuda.empty_cache()
        # One 8192-query causal prefill, bf16: the indexer and attention are MFMA-bound.
        c4 = inputs.prefill(8192, device=dev)
        legs["prefill_8192_bf16"] = bench_leg(dsa, torch, c4, 5, 2, copy_gbs,
                                              mfma_stages=("index_scores", "sparse_mla"))
        if not args.no_cpu:
            legs["prefill_8192_bf16"]["cpu_baseline"] = cpu_baseline_prefill_sample(c4)
        del c4
        torch.cuda.empty_cache()
        line["workloads"] = legs

    if not args.no_extra:
        # The per-head products on either side of the attention (decode, one row).
        line["projections"] = bench_projections(dsa, torch, 1, 1, max(20, args.steps // 4), dev)
        # The weight-free indexer input preparation (RoPE, rotation, fp8 quantisation).
        line["indexer_prep"] = bench_prep(dsa, torch, max(20, args.steps // 4), dev)
        # The MHA-form prefill attention (per-head keys and values).
        line["mha_prefill"] = bench_mha_prefill(dsa, torch, 5, dev)

    # --- sparse vs dense over context (batch 8, fp8 indexer) ---
    if not args.no_sweep:
        ctxs, sp, de = [], [], []
        for c in inputs.SWEEP_CONTEXTS:
            sc = inputs.sweep(c, device=dev)
            rs = bench_workload(dsa, torch, sc, max(20, args.steps // 4), 5, per_kernel=False,
                                replays=0)
            dm = bench_dense(dsa, torch, sc, max(20, args.steps // 4), 5)
            ctxs.append(c)
            sp.append(rs["ms_per_step"])
            de.append(dm)
            del sc
            torch.cuda.empty_cache()
        line["dense_break_even"] = {"context": break_even(ctxs, sp, de),
                                    "workload": "sweep_b8_fp8", "contexts": ctxs,
                                    "sparse_ms": [round(x, 5) for x in sp],
                                    "dense_ms": [round(x, 5) for x in de]}
        # Contexts of at most k positions keep every key, so skipping the indexer and the
        # selection (dense attention over each causal prefix) gives the same output; the
        # default path runs every stage, and this is the time such a bypass takes.
        short = [i for i, c in enumerate(ctxs) if c <= inputs.TOPK]
        line["dense_break_even"]["bypass"] = {
            "contexts": [ctxs[i] for i in short], "ms": [round(de[i], 5) for i in short],
            "full_path_ms": [round(sp[i], 5) for i in short]}
        detail["sweep"] = line["dense_break_even"]

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(host_case, args.cpu_budget)

    if args.detail:
        with open(args.detail, "w") as f:
            json.dump(detail, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
