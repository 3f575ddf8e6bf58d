#!/usr/bin/env python3
"""Benchmark of the DSA decode hot path on one MI355X.

A step is one dsa_forward call (lightning indexer -> top-2048 -> sparse
absorbed MLA) over one batch of synthetic inputs already resident in HBM.
The headline workload is batch-1 decode at 32768 cached tokens in bf16
(64x128 indexer, 128-head 512+64 MLA).  Inputs are rotated over enough
copies (>= 1 GiB in total) that every step reads its caches from HBM rather
than from the 256 MB last-level cache.

Printed: one JSON line with the throughput (query tokens/s), a roofline
entry for the dominant kernel (algorithmic bytes per launch / average launch
time, from HIP events on the launch stream), the CPU oracle timed on a
bounded sample of the same workload, and the measured sparse-vs-dense
break-even context of the batch-8 fp8 sweep.
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

# Algorithmic bytes (compulsory input reads + output writes; intermediates excluded).
def indexer_bytes(n_keys_total, rows, fp8):
    per_key = 132 if fp8 else 256            # 128-dim key (+ fp32 scale for fp8)
    per_row = (8192 + 256 + 256) if fp8 else (16384 + 256)  # q (+ q_scale) + weights
    return per_key * n_keys_total + per_row * rows


def sparse_mla_bytes(n_selected_total, rows):
    # gathered 512+64 bf16 rows, q_nope+q_pe (147456 B), bf16 output (131072 B)
    return 1152 * n_selected_total + (147456 + 131072) * rows


def dense_mla_bytes(n_keys_total, rows):
    return 1152 * n_keys_total + (147456 + 131072) * rows


def topk_bytes(n_keys_total, rows, k):
    return 4 * n_keys_total + 4 * k * rows


# The HIP kernels behind each stage of the decode step (a stage's time is the
# sum of its kernels' launch durations plus the gaps between them).
STAGE_KERNELS = {
    "index_scores": ["indexer_kernel"],
    "topk": ["topk_reset_kernel", "topk_split_kernel", "topk_finish_kernel"],
    "sparse_mla": ["mla_kernel", "mla_combine_kernel"],
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
    """Times `reps` calls of fn(i) with HIP events on the launch stream.

    The `reps` calls are captured into one HIP graph (torch.cuda.CUDAGraph),
    replayed once untimed, then once between the two events, so the timed
    region holds exactly `reps` calls and measures the GPU, not the Python
    launch loop.  Events are recorded on the stream the graph runs on.
    """

    def __init__(self, torch, graph=True):
        self.torch = torch
        self.graph = graph

    def time(self, fn, reps):
        t = self.torch
        if not self.graph:
            s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
            t.cuda.synchronize()
            s.record()
            for i in range(reps):
                fn(i)
            e.record()
            t.cuda.synchronize()
            return s.elapsed_time(e) / reps  # ms
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
        s, e = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        t.cuda.synchronize()
        return s.elapsed_time(e) / reps  # ms


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


def bench_workload(dsa, torch, case, steps, warmup, per_kernel=True):
    """Time dsa_forward (and, separately, each stage) over rotated input copies."""
    copies = rotation(case)
    B, T, S, k = case.B, case.T, case.S_max, case.topk
    dev = case.q.device
    mep = case.max_end_pos
    ws = torch.zeros(dsa.forward_workspace_size(B, T, S, k), dtype=torch.uint8, device=dev)
    out = torch.empty((B, T, 128, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, T, 128), dtype=torch.float32, device=dev)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=dev)
    scores = torch.empty((B, T, S), dtype=torch.float32, device=dev)

    def step(i):
        c = copies[i % len(copies)]
        dsa.forward(c.q, c.w, c.k_cache, c.end_pos, c.q_nope, c.q_pe, c.kv_cache, c.pe_cache,
                    c.scale, c.softmax_scale, k=k, q_scale=c.q_scale, k_scale=c.k_scale,
                    max_end_pos=mep, out=out, lse=lse, topk_out=idx, workspace=ws)

    timer = Timer(torch)
    for i in range(warmup):
        step(i)
    ms = timer.time(step, steps)
    res = {"ms_per_step": ms, "copies": len(copies)}
    if not per_kernel:
        return res

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

    reps = max(steps, 20)
    for fn in (st_index, st_topk, st_mla):
        fn(0)
    res["stage_ms"] = {"index_scores": timer.time(st_index, reps),
                       "topk": timer.time(st_topk, reps),
                       "sparse_mla": timer.time(st_mla, reps)}
    return res


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


def cpu_baseline(case, budget_s=15.0):
    """The CPU oracle (as it stands) on a bounded sample: whole decode steps of the workload."""
    import numpy as np

    import oracle
    from sparse_attention_indexer_amd import inputs
    h = {k: (None if v is None else inputs.to_numpy(v)) for k, v in
         [(n, getattr(case, n)) for n in ("q", "w", "k_cache", "q_scale", "k_scale", "end_pos",
                                           "q_nope", "q_pe", "kv_cache", "pe_cache")]}
    reps, t0 = 0, time.perf_counter()
    while True:
        s = oracle.index_scores(h["q"], h["w"], h["k_cache"], h["end_pos"], case.scale,
                                q_scale=h["q_scale"], k_scale=h["k_scale"])
        idx = oracle.topk(np.nan_to_num(s, nan=0.0), h["end_pos"], case.topk)
        oracle.mla(h["q_nope"], h["q_pe"], h["kv_cache"], h["pe_cache"], h["end_pos"],
                   case.softmax_scale, indices=idx)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= 2000:
            break
    q_tok = reps * case.B * case.T
    return {"value": q_tok / el, "unit": "query-tok/s", "cores": oracle.max_threads(),
            "kind": "oracle",
            "sample": f"{reps} whole decode step(s) of {case.name} (B={case.B}, T={case.T}, "
                      f"n={case.max_end_pos}): fp64 indexer over every key, full-sort top-"
                      f"{case.topk}, masked-softmax MLA over 128 heads; {el:.1f} s"}


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-sweep", action="store_true", help="skip the sparse-vs-dense sweep")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
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

    # --- headline: batch-1 decode at 32K, bf16 ---
    case = inputs.decode_32k(device=dev)
    r = bench_workload(dsa, torch, case, args.steps, args.warmup)
    B, T, n, k = case.B, case.T, case.max_end_pos, case.topk
    ms = r["ms_per_step"]
    value = B * T / (ms * 1e-3)
    st = r["stage_ms"]
    kbytes = {"index_scores": indexer_bytes(n * B, B * T, False),
              "topk": topk_bytes(n * B, B * T, k),
              "sparse_mla": sparse_mla_bytes(min(n, k) * B * T, B * T)}
    dom = max(st, key=st.get)
    achieved = kbytes[dom] / (st[dom] * 1e-3) / 1e9
    digest_files = {"index_scores": ["indexer.hip"], "topk": ["topk.hip"],
                    "sparse_mla": ["mla.hip"]}[dom]
    traffic = read_traffic(f"{dom}_decode_32k_bf16.pmc.txt", source_digest(digest_files))
    step_bytes = sum(kbytes[s] for s in ("index_scores", "sparse_mla"))
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
                     "traffic": traffic, "algorithmic_bytes_per_launch": kbytes[dom],
                     "avg_launch_ms": round(st[dom], 5)},
        "stage_ms": {s: round(v, 5) for s, v in st.items()},
        "step_hbm_frac": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
    }
    detail = {"headline": r}
    # The per-head products on either side of the attention (decode, one row).
    line["projections"] = bench_projections(dsa, torch, B, T, max(20, args.steps // 4), dev)
    # The weight-free indexer input preparation (RoPE, rotation, fp8 quantisation).
    line["indexer_prep"] = bench_prep(dsa, torch, max(20, args.steps // 4), dev)
    # The MHA-form prefill attention (per-head keys and values).
    line["mha_prefill"] = bench_mha_prefill(dsa, torch, 5, dev)

    # --- sparse vs dense over context (batch 8, fp8 indexer) ---
    if not args.no_sweep:
        ctxs, sp, de = [], [], []
        for c in inputs.SWEEP_CONTEXTS:
            sc = inputs.sweep(c, device=dev)
            rs = bench_workload(dsa, torch, sc, max(20, args.steps // 4), 5, per_kernel=False)
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
        detail["sweep"] = line["dense_break_even"]

    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(case.to("cpu"), args.cpu_budget)

    if args.detail:
        with open(args.detail, "w") as f:
            json.dump(detail, f, indent=1)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
