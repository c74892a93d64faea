"""Benchmark of the ADA decode step on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload 2|3|...] [--splits S] [--layers L]

A step is one ada_decode call over the workload: the page stream (code
tables, logits, online softmax, PV) and the split merge, for every
(sequence, query head).  The cache is built on the GPU
(encode + pack) before timing; the timed region replays a HIP graph of
steps over rotated copies of the page arena, so repeated steps read HBM and
not the 256 MiB Infinity Cache.  `value` is context tokens per second of
whole steps.  The roofline entry is for the dominant kernel, the page
stream, timed alone with events on its stream.  Prints one JSON line.
With --layers L above 1 (the 32-layer workload), a step is L back-to-back
ada_decode calls over L per-layer caches, and `value` counts layer-tokens.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import compressed_kv_attention_amd as ada  # noqa: E402
import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
ROTATE_BYTES = 512 << 20  # at least this much distinct cache data per replay cycle


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_layer(cfg, layer, dev, dense=False):
    """Generates one layer's inputs and builds its caches on the GPU."""
    lens = synth.seq_lens(cfg)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    H, D = cfg.num_kv_heads, cfg.head_dim
    geom = ada.Geom(D, cfg.num_q_heads, H)
    gen_dev = "cpu" if cfg.number <= 2 else dev
    keys = synth.keys(cfg, layer, N, gen_dev).to(dev)
    vals = synth.values(cfg, layer, N, gen_dev).to(dev)
    scores = synth.scores(cfg, layer, N).to(dev)
    q = synth.queries(cfg, layer, gen_dev).to(dev)
    cb8, cb4 = (t.to(dev) for t in synth.codebooks(cfg, layer))
    bp = synth.tier_mix(cfg)
    r = torch.empty((N, H), dtype=torch.float16, device=dev)
    c8 = torch.empty((N, H, D // 8), dtype=torch.uint8, device=dev)
    c4 = torch.empty((N, H, D // 16), dtype=torch.uint8, device=dev)
    ada.encode(geom, keys, cb8, cb4, r, c8, c4)
    n_pages = ada.pack_num_pages(geom, cu, bp)
    maxp = int(max(lens)) // 16 + 4
    stored = 0
    for s in range(cfg.num_seqs):
        T = int(lens[s])
        n = [(int(bp[s][k]) * T + 5000) // 10000 for k in range(3)]
        cnt = [n[0], n[1] - n[0], n[2] - n[1]]
        stored += H * sum((c + 15) // 16 * ada.page_bytes(D, k) for k, c in enumerate(cnt))
    cache = ada.Cache(geom, cfg.num_seqs, maxp, stored)
    ada.rdr_pack(geom, cache, cu, bp, keys, vals, r, c8, c4, scores,
                 place_perm=synth.place_perm(cfg, layer, n_pages))
    out = dict(geom=geom, cache=cache, cb8=cb8, cb4=cb4, q=q, lens=lens, cu=cu, N=N)
    if dense:
        dpages = H * sum((int(T) + 15) // 16 for T in lens)
        dcache = ada.Cache(geom, cfg.num_seqs, maxp, dpages * ada.page_bytes(D, 3))
        ada.dense_pack(geom, dcache, cu, keys, vals)
        out["dense"] = dcache
    torch.cuda.synchronize()
    del keys, vals, scores, r, c8, c4
    return out


def time_eager(step_fns, steps, warmup):
    """Eager launches, events around the whole run."""
    for i in range(warmup):
        step_fns[i % len(step_fns)]()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for i in range(steps):
        step_fns[i % len(step_fns)]()
    e1.record()
    torch.cuda.synchronize()
    return steps, time.perf_counter() - t0, e0.elapsed_time(e1) / steps


def time_graph(step_fns, steps, warmup):
    """Captures one call of every fn in step_fns into a graph, replays it
    enough times for `steps` steps; returns (steps run, seconds, per-step ms
    from events)."""
    for f in step_fns:  # eager warm-up (also sets kernel attributes)
        f()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for f in step_fns:
                f()
    torch.cuda.synchronize()
    reps = max(1, math.ceil(steps / len(step_fns)))
    wreps = max(1, math.ceil(warmup / len(step_fns)))
    for _ in range(wreps):
        g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    n = reps * len(step_fns)
    return n, wall, e0.elapsed_time(e1) / n


def batch_event_ms(step_fns, n):
    """Mean duration of n back-to-back launches (the GPU stays busy: each
    launch is queued well before the previous one ends), from two events on
    the launch stream around the batch."""
    st = torch.cuda.current_stream()
    for f in step_fns:
        f()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(st)
    for i in range(n):
        step_fns[i % len(step_fns)]()
    e1.record(st)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def kernel_event_ms(step_fns, n):
    """Average duration of single decode launches, each bracketed by events
    on the launch stream (eager launches; the GPU timestamps the events)."""
    st = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i in range(n):
        evs[i][0].record(st)
        step_fns[i % len(step_fns)]()
        evs[i][1].record(st)
    torch.cuda.synchronize()
    ts = sorted(a.elapsed_time(b) for a, b in evs)
    return float(np.median(ts)), float(np.mean(ts))


def cpu_threads():
    """Threads the oracle runs on: the cores this process may use (its CPU
    affinity), capped by OMP_NUM_THREADS where the machine sets it."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    return max(1, min(n, int(cap))) if cap.isdigit() and int(cap) > 0 else max(1, n)


def cpu_baseline(cfg, layer, seconds_target=10.0):
    """The CPU oracle (test infrastructure) timed on this host on a bounded
    sample: whole decode steps of the same workload on oracle-built pages,
    on every usable core and on one, plus oracle encode of the workload's
    keys and of the 32-layer workload's 512-token append chunk (one layer)."""
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import oracle
    lens = synth.seq_lens(cfg)
    if cfg.number > 2:
        return None
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    keys = synth.keys(cfg, layer, N)
    vals = synth.values(cfg, layer, N)
    scores = synth.scores(cfg, layer, N)
    q = synth.queries(cfg, layer)
    cb8, cb4 = synth.codebooks(cfg, layer)
    threads = cpu_threads()
    t0 = time.perf_counter()
    r, c8, c4 = oracle.encode(keys, cb8, cb4, nthreads=threads)
    t_enc = time.perf_counter() - t0
    hc = oracle.HostCache(cfg.head_dim, cfg.num_kv_heads, cfg.num_seqs, int(max(lens)) // 16 + 4,
                          N * cfg.num_kv_heads * 512 + (1 << 20), slot_tokens=False)
    assert oracle.pack(hc, cu, synth.tier_mix(cfg), keys, vals, r, c8, c4, scores) == 0
    units = cfg.num_seqs * cfg.num_q_heads
    dthreads = min(threads, units)
    reps, t = 0, 0.0
    res = None
    while t < seconds_target and reps < 50:
        t0 = time.perf_counter()
        res = oracle.decode(hc, cb8, cb4, q, cfg.sigma, nthreads=dthreads)
        t += time.perf_counter() - t0
        reps += 1
    # one thread, one whole step
    t0 = time.perf_counter()
    oracle.decode(hc, cb8, cb4, q, cfg.sigma, nthreads=1)
    t1 = time.perf_counter() - t0
    # encode of one layer's append chunk of the 32-layer workload
    c5 = synth.WORKLOADS[5]
    na = c5.num_seqs * c5.append_tokens
    ak = synth.keys(c5, 0, na, stream="k-append")
    a8, a4 = synth.codebooks(c5, 0)
    t0 = time.perf_counter()
    oracle.encode(ak, a8, a4, nthreads=threads)
    t_app = time.perf_counter() - t0
    tokens = int(lens.sum())
    return dict(value=tokens * reps / t, unit="KV tokens/s", cores=dthreads, kind="oracle",
                host_logical_cpus=os.cpu_count(), usable_cpus=threads,
                sample=f"{reps} whole decode steps of the workload (all {units} query heads, "
                       f"T={tokens}), double precision, {dthreads} threads",
                single_thread_value=tokens / t1,
                encode_token_heads_per_s=N * cfg.num_kv_heads / t_enc,
                encode_seconds=t_enc,
                append_chunk_encode_seconds=t_app,
                append_chunk=f"{c5.name}: {c5.append_tokens} tokens x {c5.num_seqs} sequences x "
                             f"{c5.num_kv_heads} heads, one layer, {threads} threads"), res


def append_path(dev, reps=20):
    """Times the append path on the 32-layer workload's shape: ada_encode and
    rdr_pack of 512 new tokens for each of 8 sequences (one layer), into a
    cache that already holds a first chunk of those sequences."""
    cfg = synth.WORKLOADS[5]
    S, H, D, n = cfg.num_seqs, cfg.num_kv_heads, cfg.head_dim, cfg.append_tokens
    geom = ada.Geom(D, cfg.num_q_heads, H)
    cb8, cb4 = (t.to(dev) for t in synth.codebooks(cfg, 0))
    bp = synth.tier_mix(cfg)
    cu = synth.cu_tokens(np.full(S, n, np.int64))
    keys = synth.keys(cfg, 0, S * n, dev, stream="k-append")
    vals = synth.values(cfg, 0, S * n, dev, stream="v-append")
    scores = synth.scores(cfg, 0, S * n, stream="score-append").to(dev)
    r = torch.empty((S * n, H), dtype=torch.float16, device=dev)
    c8 = torch.empty((S * n, H, D // 8), dtype=torch.uint8, device=dev)
    c4 = torch.empty((S * n, H, D // 16), dtype=torch.uint8, device=dev)
    per_call = S * H * (n // 16 + 3) * ada.page_bytes(D, 0)  # a bound: every page at the largest size
    calls = 3 * reps + 2  # the ranked path, then the budget-solver path (host plan, device plan)
    cache = ada.Cache(geom, S, calls * (n // 16 + 3), per_call * calls)
    ws = torch.zeros(ada.pack_workspace_size(geom, S * n, S), dtype=torch.uint8, device=dev)
    pos = np.zeros(S, np.int64)
    ada.encode(geom, keys, cb8, cb4, r, c8, c4)
    ada.rdr_pack(geom, cache, cu, bp, keys, vals, r, c8, c4, scores, pos_base=pos, ws=ws)
    torch.cuda.synchronize()
    e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    enc, pack = 0.0, 0.0
    for i in range(reps):
        pos += n
        e[0].record()
        ada.encode(geom, keys, cb8, cb4, r, c8, c4)
        e[1].record()
        ada.rdr_pack(geom, cache, cu, bp, keys, vals, r, c8, c4, scores, pos_base=pos, ws=ws)
        e[2].record()
        torch.cuda.synchronize()
        enc += e[0].elapsed_time(e[1])
        pack += e[1].elapsed_time(e[2])
    th = S * n * H
    res = {"workload": f"{cfg.name} append, one layer", "tokens": S * n, "token_heads": th,
           "encode_us": enc / reps * 1e3, "pack_us": pack / reps * 1e3,
           "token_heads_per_s": th / ((enc + pack) / reps / 1e3),
           "note": "pack includes its host plan and the plan's host-to-device copy"}
    # the same append with the budget solver choosing the tiers (60% budget)
    e8 = torch.empty((S * n, H), device=dev)
    e4 = torch.empty((S * n, H), device=dev)
    tiers = torch.empty((S * n, H), dtype=torch.uint8, device=dev)
    budgets = synth.budget_bytes(cfg, np.full(S, n, np.int64))
    sws = torch.zeros(ada.solve_workspace_size(geom, S, S * n), dtype=torch.uint8, device=dev)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    t = np.zeros(5)
    for i in range(reps):
        pos += n
        e[0].record()
        ada.encode(geom, keys, cb8, cb4, r, c8, c4)
        e[1].record()
        ada.code_error(geom, keys, cb8, cb4, c8, c4, e8, e4)
        e[2].record()
        ada.rdr_solve(geom, cu, budgets, r, e8, e4, scores, tiers, ws=sws)
        e[3].record()
        counts = ada.tier_counts(geom, cu, tiers)
        e[4].record()
        ada.rdr_pack_tiers(geom, cache, cu, counts, tiers, keys, vals, r, c8, c4, pos_base=pos, ws=ws)
        e[5].record()
        torch.cuda.synchronize()
        t += [e[k].elapsed_time(e[k + 1]) for k in range(5)]
    t = t / reps * 1e3
    res["solver"] = {"budget_bp": int(synth.budgets_bp(cfg)[0]), "encode_us": t[0], "code_error_us": t[1],
                     "solve_us": t[2], "tier_counts_us": t[3], "pack_tiers_us": t[4],
                     "token_heads_per_s": th / (t.sum() / 1e6),
                     "note": "tier_counts includes its device-to-host copy and stream synchronization"}
    # the same chain with the page plan made on the device: no host round
    # trip, so the whole chain is enqueued at once and timed end to end
    state = ada.AppendState(geom, cache)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        pos += n
        ada.encode(geom, keys, cb8, cb4, r, c8, c4)
        ada.code_error(geom, keys, cb8, cb4, c8, c4, e8, e4)
        ada.rdr_solve(geom, cu, budgets, r, e8, e4, scores, tiers, ws=sws)
        ada.rdr_pack_tiers_device(geom, cache, state, cu, tiers, keys, vals, r, c8, c4, pos_base=pos, ws=ws)
    e1.record()
    torch.cuda.synchronize()
    status = state.pull()
    chain_us = e0.elapsed_time(e1) / reps * 1e3
    res["solver_device_plan"] = {"chain_us": chain_us, "token_heads_per_s": th / (chain_us / 1e6),
                                 "status": status,
                                 "note": "encode, code error, solve and rdr_pack_tiers_device per chunk, "
                                         "enqueued back to back with no synchronization"}
    return res


def append_steps(dev, steps=200):
    """Times the decode-step append (ada_append) on the 32-layer workload's
    shape: one new token for each of 8 sequences x 8 KV heads (one layer),
    tiered by the slope thresholds of a budget solve over a 512-token
    chunk, captured once in a graph and replayed."""
    cfg = synth.WORKLOADS[5]
    S, H, D, n = cfg.num_seqs, cfg.num_kv_heads, cfg.head_dim, cfg.append_tokens
    geom = ada.Geom(D, cfg.num_q_heads, H)
    cb8, cb4 = (t.to(dev) for t in synth.codebooks(cfg, 0))
    cu = synth.cu_tokens(np.full(S, n, np.int64))
    keys = synth.keys(cfg, 0, S * n, dev, stream="k-append")
    scores = synth.scores(cfg, 0, S * n, stream="score-append").to(dev)
    r = torch.empty((S * n, H), dtype=torch.float16, device=dev)
    c8 = torch.empty((S * n, H, D // 8), dtype=torch.uint8, device=dev)
    c4 = torch.empty((S * n, H, D // 16), dtype=torch.uint8, device=dev)
    ada.encode(geom, keys, cb8, cb4, r, c8, c4)
    e8 = torch.empty((S * n, H), device=dev)
    e4 = torch.empty((S * n, H), device=dev)
    ada.code_error(geom, keys, cb8, cb4, c8, c4, e8, e4)
    tiers = torch.empty((S * n, H), dtype=torch.uint8, device=dev)
    th = torch.empty(S, device=dev)
    ada.rdr_solve(geom, cu, synth.budget_bytes(cfg, np.full(S, n, np.int64)), r, e8, e4, scores, tiers,
                  threshold=th)
    maxp = (steps + 50) // 16 + 8
    cache = ada.Cache(geom, S, maxp, S * H * maxp * ada.page_bytes(D, 0))
    state = ada.AppendState(geom, cache)
    kb = synth.keys(cfg, 0, S, dev, stream="k-step").contiguous()
    vb = synth.values(cfg, 0, S, dev, stream="v-step").contiguous()
    sb = synth.scores(cfg, 0, S, stream="s-step").to(dev)
    pb = torch.zeros(S, dtype=torch.int64, device=dev)
    per_graph = 50  # steps captured in one graph, so host launch cost does not count
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(per_graph):
            ada.append(geom, cache, state, cb8, cb4, kb, vb, sb, th, pb)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps // per_graph):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    status = state.pull()
    n = steps // per_graph * per_graph
    return {"workload": f"{cfg.name}: one token x {S} sequences x {H} heads per step, one layer",
            "steps": n, "us_per_step": e0.elapsed_time(e1) / n * 1e3, "status": status,
            "pages": int(cache.num_pages_host.sum()),
            "note": f"graphs of {per_graph} ada_append launches replayed back to back (the same token each step)"}


def solver_full(cfg, dev, reps=5):
    """Times the budget solver over a whole workload (one layer): code error,
    solve, tier counts and tier-given pack of every token."""
    S, H, D = cfg.num_seqs, cfg.num_kv_heads, cfg.head_dim
    geom = ada.Geom(D, cfg.num_q_heads, H)
    lens = synth.seq_lens(cfg)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    keys = synth.keys(cfg, 0, N, dev)
    vals = synth.values(cfg, 0, N, dev)
    scores = synth.scores(cfg, 0, N).to(dev)
    cb8, cb4 = (t.to(dev) for t in synth.codebooks(cfg, 0))
    r = torch.empty((N, H), dtype=torch.float16, device=dev)
    c8 = torch.empty((N, H, D // 8), dtype=torch.uint8, device=dev)
    c4 = torch.empty((N, H, D // 16), dtype=torch.uint8, device=dev)
    ada.encode(geom, keys, cb8, cb4, r, c8, c4)
    e8 = torch.empty((N, H), device=dev)
    e4 = torch.empty((N, H), device=dev)
    tiers = torch.empty((N, H), dtype=torch.uint8, device=dev)
    budgets = synth.budget_bytes(cfg, lens)
    sws = torch.zeros(ada.solve_workspace_size(geom, S, N), dtype=torch.uint8, device=dev)
    pws = torch.zeros(ada.pack_workspace_size(geom, N, S), dtype=torch.uint8, device=dev)
    e = [torch.cuda.Event(enable_timing=True) for _ in range(6)]
    t = np.zeros(4)
    stored = 0
    for i in range(reps + 1):
        e[0].record()
        ada.code_error(geom, keys, cb8, cb4, c8, c4, e8, e4)
        e[1].record()
        ada.rdr_solve(geom, cu, budgets, r, e8, e4, scores, tiers, ws=sws)
        e[2].record()
        counts = ada.tier_counts(geom, cu, tiers)
        e[3].record()
        stored = sum(ada.page_bytes(D, k) * ((counts[:, k] + 15) // 16).sum() for k in range(3))
        cache = ada.Cache(geom, S, int(max(lens)) // 16 + 4, int(stored))
        torch.cuda.synchronize()
        e[4].record()
        ada.rdr_pack_tiers(geom, cache, cu, counts, tiers, keys, vals, r, c8, c4, ws=pws)
        e[5].record()
        torch.cuda.synchronize()
        if i > 0:  # the first round warms up
            t += [e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2]), e[2].elapsed_time(e[3]),
                  e[4].elapsed_time(e[5])]
        del cache
    t = t / reps * 1e3
    th = N * H
    mix = np.bincount(tiers.cpu().numpy().ravel(), minlength=4) / th
    dense = int(np.asarray(lens, np.int64).sum()) * H * 4 * D
    return {"workload": cfg.name, "token_heads": th, "budget_bp": [int(x) for x in np.unique(synth.budgets_bp(cfg))][:4],
            "code_error_us": t[0], "solve_us": t[1], "tier_counts_us": t[2], "pack_tiers_us": t[3],
            "solve_token_heads_per_s": th / (t[1] / 1e6), "tier_mix": [round(float(x), 4) for x in mix],
            "stored_fraction_of_dense": stored / dense,
            "note": "tier_counts includes its device-to-host copy and stream synchronization; "
                    "pack_tiers its host plan and the plan's copy"}


def stream_bytes(L):
    """Bytes the page-stream kernel must read from HBM per launch: the stored
    pages and their page-table entries (4 B offset + 1 B metadata)."""
    cache = L["cache"]
    return cache.used_bytes() + int(cache.num_pages_host.sum()) * 5


def profiled_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    rocprofv3 counter summary, if that summary was taken on the current
    kernel source; else None."""
    import glob
    import hashlib
    src = os.path.join(ROOT, "compressed_kv_attention_amd", "csrc", "decode.hip")
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    for f in sorted(glob.glob(os.path.join(ROOT, "profiles", "*.md"))):
        for line in open(f):
            if line.startswith("traffic: "):
                rec = json.loads(line[len("traffic: "):])
                if rec.get("kernel") == kernel and rec.get("workload") == workload:
                    return rec["bytes_per_launch"] if rec.get("source_sha256") == sha else None
    return None


def algorithmic_bytes(L, cfg):
    """Bytes one decode step must move: stored pages, codebooks, page table
    and metadata, queries, outputs."""
    cache = L["cache"]
    pages = int(cache.num_pages_host.sum())
    G = cfg.head_dim // 8
    cb = cfg.num_kv_heads * G * (256 + 16) * 8 * 4
    qb = cfg.num_seqs * cfg.num_q_heads * cfg.head_dim * 2
    ob = cfg.num_seqs * cfg.num_q_heads * (cfg.head_dim + 1) * 4
    return cache.used_bytes() + cb + pages * 5 + qb + ob


def multi_layer(cfg, layers, dev, steps, warmup, eager):
    """A whole-model attention step: `layers` layers' caches built one after
    another (per-layer codebooks, keys, values and queries), and one step =
    back-to-back ada_decode calls over every layer on one stream.  The
    layers' pages together far exceed the last-level cache, so no copies
    are rotated."""
    Ls = []
    t0 = time.perf_counter()
    for layer in range(layers):
        Ls.append(build_layer(cfg, layer, dev))
        if layer % 8 == 7 or layer == layers - 1:
            log(f"built layer {layer + 1}/{layers} ({time.perf_counter() - t0:.1f} s)")
    geom = Ls[0]["geom"]
    S, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    maxp = max(L["cache"].maxp for L in Ls)
    outs = [torch.empty((S, Hq, D), device=dev) for _ in Ls]
    lses = [torch.empty((S, Hq), device=dev) for _ in Ls]
    out, lse = outs[0], lses[0]
    ws = torch.zeros(ada.decode_workspace_size(geom, S, maxp, 0), dtype=torch.uint8, device=dev)

    def step():
        for L, o, l in zip(Ls, outs, lses):
            ada.decode(geom, L["cache"], L["cb8"], L["cb4"], L["q"], cfg.sigma, o, l, ws=ws)

    timer = time_eager if eager else time_graph
    n, _, ms = timer([step], steps, warmup)
    tokens = int(Ls[0]["lens"].sum()) * layers
    used = sum(L["cache"].used_bytes() for L in Ls)
    alg = sum(algorithmic_bytes(L, cfg) for L in Ls)
    sfns = [(lambda L=L: ada.decode_stage("stream", geom, L["cache"], L["cb8"], L["cb4"], L["q"],
                                          cfg.sigma, out, lse, ws=ws)) for L in Ls]
    k_mean = batch_event_ms(sfns, 2 * layers)
    sbytes = sum(stream_bytes(L) for L in Ls) / layers
    achieved = sbytes / (k_mean / 1e3) / 1e9
    log(f"{layers}-layer step {ms:.3f} ms (graph); page stream {k_mean * 1e3:.2f} us per layer, "
        f"{achieved:.0f} GB/s")
    return {
        "metric": "ADA decode KV tokens/s per step",
        "value": tokens / (ms / 1e3),
        "unit": "KV layer-tokens/s",
        "n_gpus": 1, "steps": n, "warmup": warmup, "ms_per_step": ms,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp32", "data": "synthetic",
        "config": {"workload": cfg.name, "layers": layers, "num_seqs": S,
                   "seq_len": int(Ls[0]["lens"].max()), "layer_tokens_per_step": tokens,
                   "num_q_heads": Hq, "num_kv_heads": cfg.num_kv_heads, "head_dim": D,
                   "tier_cum_bp": list(map(int, synth.tier_mix(cfg)[0])),
                   "splits": ada.decode_default_splits(geom, S, maxp)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": None,
                     "kernel": f"decode_main<{D},{Hq // cfg.num_kv_heads},false>",
                     "kernel_us_mean": k_mean * 1e3, "bytes_per_launch": sbytes},
        "step_roofline": {"bytes_per_step": alg, "achieved_GBs": alg / (ms / 1e3) / 1e9,
                          "frac": alg / (ms / 1e3) / 1e9 / HBM_PEAK_GBS},
        "stored_bytes": used,
        "stored_fraction_of_dense": used / (tokens * cfg.num_kv_heads * 4 * D),
    }


def measure_step(cfg, L, args, out, lse, ws, timer):
    """Times whole decode steps of one built layer (graph replays over rotated
    arena copies) and the page-stream kernel alone (events around
    back-to-back launches on its stream)."""
    geom, cache = L["geom"], L["cache"]
    S, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    used = cache.used_bytes()
    n_copies = max(2, math.ceil(ROTATE_BYTES / max(used, 1)) + 1)
    arenas = [cache.arena] + [cache.arena.clone() for _ in range(n_copies - 1)]
    views = [cache.view(a) for a in arenas]
    splits = args.splits or ada.decode_default_splits(geom, S, cache.maxp)

    def make_step(v):
        return lambda: ada.decode(geom, cache, L["cb8"], L["cb4"], L["q"], cfg.sigma, out, lse,
                                  num_splits=args.splits, ws=ws, view=v)

    fns = [make_step(v) for v in views]
    log(f"{cfg.name}: stored {used / 1e6:.2f} MB in {int(cache.num_pages_host.sum())} pages; "
        f"{n_copies} arena copies; {splits} splits per row")
    steps, _, ms_graph = timer(fns, args.steps, args.warmup)
    tokens = int(L["lens"].sum())
    alg = algorithmic_bytes(L, cfg)

    def make_stream(v):
        return lambda: ada.decode_stage("stream", geom, cache, L["cb8"], L["cb4"], L["q"], cfg.sigma,
                                        out, lse, num_splits=args.splits, ws=ws, view=v)

    sfns = [make_stream(v) for v in views]
    k_mean = batch_event_ms(sfns, max(200, 4 * n_copies))
    k_med, _ = kernel_event_ms(sfns, max(50, 2 * n_copies))
    sbytes = stream_bytes(L)
    achieved = sbytes / (k_mean / 1e3) / 1e9
    kernel_name = f"decode_main<{D},{Hq // cfg.num_kv_heads},false>"
    traffic = profiled_traffic(kernel_name, cfg.name)
    log(f"{cfg.name}: step {ms_graph * 1e3:.2f} us (graph); page stream {k_mean * 1e3:.2f} us mean of "
        f"back-to-back launches, {k_med * 1e3:.2f} us median single launch (events), {achieved:.0f} GB/s")
    return {
        "value": tokens / (ms_graph / 1e3), "unit": "KV tokens/s", "steps": steps, "ms_per_step": ms_graph,
        "config": {"workload": cfg.name, "num_seqs": S, "seq_len": int(L["lens"].max()),
                   "tokens_per_step": tokens, "num_q_heads": Hq, "num_kv_heads": cfg.num_kv_heads,
                   "head_dim": D, "tier_cum_bp": list(map(int, synth.tier_mix(cfg)[0])),
                   "splits": splits, "arena_copies": n_copies},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": achieved / HBM_PEAK_GBS, "traffic": traffic,
                     "kernel": kernel_name, "kernel_us_mean": k_mean * 1e3,
                     "kernel_us_median_single_launch": k_med * 1e3, "bytes_per_launch": sbytes},
        "step_roofline": {"bytes_per_step": alg, "achieved_GBs": alg / (ms_graph / 1e3) / 1e9,
                          "frac": alg / (ms_graph / 1e3) / 1e9 / HBM_PEAK_GBS},
        "stored_bytes": used,
        "stored_fraction_of_dense": used / (tokens * cfg.num_kv_heads * 4 * D),
        "_views": views,
    }


def phase_profile(cfg, dev, args):
    """Per-wave phase timestamps of the page stream (the tracing build,
    ada_phase_trace) for the last step of graph replays over rotated arena
    copies, as the step is timed.  Durations in microseconds; percentiles
    0/10/50/90/100 over all waves (or blocks) of the launch."""
    log(f"workload {cfg.number} {cfg.name}: building cache on the GPU (tracing build)")
    L = build_layer(cfg, 0, dev)
    geom, cache = L["geom"], L["cache"]
    S, Hq, D, H = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim, cfg.num_kv_heads
    out = torch.empty((S, Hq, D), device=dev)
    lse = torch.empty((S, Hq), device=dev)
    ws = torch.zeros(ada.decode_workspace_size(geom, S, cache.maxp, args.splits), dtype=torch.uint8, device=dev)
    splits = args.splits or ada.decode_default_splits(geom, S, cache.maxp)
    waves = 8 if (D == 128 and Hq // H > 4) else 12
    nblk = S * H * splits
    trace = torch.zeros(nblk * waves * 8, dtype=torch.int64, device=dev)
    n_copies = max(2, math.ceil(ROTATE_BYTES / max(cache.used_bytes(), 1)) + 1)
    views = [cache.view(a) for a in [cache.arena] + [cache.arena.clone() for _ in range(n_copies - 1)]]
    fns = [(lambda v=v: ada.decode(geom, cache, L["cb8"], L["cb4"], L["q"], cfg.sigma, out, lse,
                                   num_splits=args.splits, ws=ws, view=v)) for v in views]
    ada.phase_trace(trace)
    steps, _, ms = time_graph(fns, args.steps, args.warmup)
    torch.cuda.synchronize()
    ada.phase_trace(None)
    t = trace.view(nblk, waves, 8).cpu().numpy()
    ts = t[:, :, :6].astype(np.int64)
    rel = (ts - ts[:, :, 0].min()) / 100.0  # 100 MHz ticks -> us

    def pct(x):
        return [round(float(np.percentile(x, q)), 2) for q in (0, 10, 50, 90, 100)]

    names = ["prologue_loads", "table_build", "table_barrier_wait", "page_loop", "epilogue"]
    res = {"workload": cfg.name, "splits": splits, "blocks": nblk, "waves_per_block": waves,
           "arena_copies": n_copies, "step_us_tracing_build": ms * 1e3,
           "per_wave_us": {n: pct(rel[:, :, k + 1] - rel[:, :, k]) for k, n in enumerate(names)},
           "block_start_us": pct(rel[:, :, 0].min(1)),
           "block_past_table_barrier_us": pct(rel[:, :, 3].max(1)),
           "block_end_us": pct(rel[:, :, 5].max(1)),
           "block_end_us_by_xcc": {int(x): pct(rel[:, :, 5].max(1)[(t[:, 0, 7] & 7) == x])
                                   for x in range(8) if ((t[:, 0, 7] & 7) == x).any()},
           "xcc_of_block0": int(t[0, 0, 7] & 7),
           "xcc_round_robin_fraction": float(np.mean((t[:, 0, 7] & 7) == ((np.arange(nblk) + int(t[0, 0, 7] & 7)) % 8)))}
    return res


def second_context_length(number, dev, args, timer):
    """The same measurement on a second workload (the long-context batch by
    default), reported beside the headline in the same line."""
    cfg = synth.WORKLOADS[number]
    log(f"workload {cfg.number} {cfg.name}: building cache on the GPU")
    L = build_layer(cfg, 0, dev)
    S, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    out = torch.empty((S, Hq, D), device=dev)
    lse = torch.empty((S, Hq), device=dev)
    ws = torch.zeros(ada.decode_workspace_size(L["geom"], S, L["cache"].maxp, args.splits),
                     dtype=torch.uint8, device=dev)
    m = measure_step(cfg, L, args, out, lse, ws, timer)
    m.pop("_views")
    del L
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return m


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--layers", type=int, default=1,
                    help="layers per step (each with its own cache); above 1 times the whole "
                         "multi-layer step only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-append", action="store_true", help="skip the append-path timing")
    ap.add_argument("--no-sym", action="store_true", help="skip the symmetric-variant timing")
    ap.add_argument("--solver-full", action="store_true",
                    help="also time the budget solver over the whole workload")
    ap.add_argument("--eager", action="store_true",
                    help="time eager launches instead of graph replays (for profilers)")
    ap.add_argument("--second-workload", type=int, default=3,
                    help="workload measured beside the headline in the same line (0 = none): "
                         "by default the 4 x 131072-token batch, the other context length the "
                         "metric is quoted at")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run one device-to-device copy of this size first (counter calibration)")
    ap.add_argument("--phase-trace", action="store_true",
                    help="print the page stream's per-wave phase timestamps instead of the bench "
                         "line (needs libada_trace.so: python -m compressed_kv_attention_amd.build "
                         "--phase-trace)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the ADA decode path has no multi-GPU mode "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.phase_trace:
        ada.use_tracing_build()
    ada.load()
    cfg = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    if args.phase_trace:
        print(json.dumps(phase_profile(cfg, dev, args)))
        return
    if args.layers > 1:
        if args.layers > cfg.num_layers:
            print(f"workload {cfg.number} has {cfg.num_layers} layer(s)", file=sys.stderr)
            sys.exit(2)
        print(json.dumps(multi_layer(cfg, args.layers, dev, args.steps, args.warmup, args.eager)))
        return
    if args.copy_probe_mib:
        src = torch.ones(args.copy_probe_mib << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy probe: {args.copy_probe_mib} MiB device-to-device")
        del src, dst
    log(f"workload {cfg.number} {cfg.name}: building cache on the GPU")
    L = build_layer(cfg, 0, dev, dense=not args.no_dense)
    geom, cache = L["geom"], L["cache"]
    S, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    out = torch.empty((S, Hq, D), device=dev)
    lse = torch.empty((S, Hq), device=dev)
    ws = torch.zeros(ada.decode_workspace_size(geom, S, cache.maxp, args.splits), dtype=torch.uint8,
                     device=dev)
    timer = time_eager if args.eager else time_graph
    m = measure_step(cfg, L, args, out, lse, ws, timer)
    # (each view keeps its arena copy alive: the copies must outlive every
    # call below that reads them, the symmetric variant's included)
    views, n_copies = m.pop("_views"), m["config"]["arena_copies"]
    tokens = m["config"]["tokens_per_step"]
    ms_graph = m["ms_per_step"]
    result = {
        "metric": "ADA decode KV tokens/s per step",
        "value": m["value"],
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": m["steps"],
        "warmup": args.warmup,
        "ms_per_step": ms_graph,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "data": "synthetic",
        "config": m["config"],
        "roofline": m["roofline"],
        "step_roofline": m["step_roofline"],
        "stored_bytes": m["stored_bytes"],
        "stored_fraction_of_dense": m["stored_fraction_of_dense"],
    }
    if "dense" in L:
        dc = L["dense"]
        dused = dc.used_bytes()
        dcop = max(2, math.ceil(ROTATE_BYTES / dused) + 1)
        darenas = [dc.arena] + [dc.arena.clone() for _ in range(dcop - 1)]
        dws = torch.zeros(ada.decode_workspace_size(geom, S, dc.maxp, args.splits), dtype=torch.uint8,
                          device=dev)
        dfns = [(lambda v=dc.view(a): ada.dense_decode(geom, dc, L["q"], cfg.sigma, out, lse,
                                                      num_splits=args.splits, ws=dws, view=v))
                for a in darenas]
        _, _, dms = timer(dfns, args.steps, args.warmup)
        result["dense_bf16_baseline"] = {"ms_per_step": dms, "value": tokens / (dms / 1e3),
                                         "stored_bytes": dused,
                                         "achieved_GBs": dused / (dms / 1e3) / 1e9,
                                         "ada_speedup": dms / ms_graph}
        del darenas
    if not args.no_sym:
        # the symmetric angle-code variant on the same cache
        yws = torch.zeros(ada.decode_sym_workspace_size(geom, S, cache.maxp, args.splits), dtype=torch.uint8,
                          device=dev)
        yfns = [(lambda v=v: ada.decode_sym(geom, cache, L["cb8"], L["cb4"], L["q"], cfg.sigma, out, lse,
                                            num_splits=args.splits, ws=yws, view=v)) for v in views]
        _, _, yms = timer(yfns, args.steps, args.warmup)
        result["symmetric_variant"] = {"ms_per_step": yms, "value": tokens / (yms / 1e3),
                                       "note": "ada_decode_sym: query codes and table kernel, page stream, merge"}
        log(f"symmetric variant: step {yms * 1e3:.2f} us")
    torch.cuda.synchronize()
    if not args.no_append:
        result["append_path"] = append_path(dev)
        ap = result["append_path"]
        log(f"append path: encode {ap['encode_us']:.1f} us, pack {ap['pack_us']:.1f} us per layer; "
            f"with the budget solver: code error {ap['solver']['code_error_us']:.1f} us, "
            f"solve {ap['solver']['solve_us']:.1f} us, counts {ap['solver']['tier_counts_us']:.1f} us, "
            f"pack {ap['solver']['pack_tiers_us']:.1f} us; with the device page plan the chain takes "
            f"{ap['solver_device_plan']['chain_us']:.1f} us")
    if not args.no_append:
        result["append_step"] = append_steps(dev)
        log(f"decode-step append: {result['append_step']['us_per_step']:.2f} us per step "
            f"(64 token-heads, graph replay)")
    if args.solver_full:
        result["solver_full"] = solver_full(cfg, dev)
        sf = result["solver_full"]
        log(f"budget solver over the workload: code error {sf['code_error_us']:.1f} us, "
            f"solve {sf['solve_us']:.1f} us, counts {sf['tier_counts_us']:.1f} us, "
            f"pack {sf['pack_tiers_us']:.1f} us; mix {sf['tier_mix']}")
    if args.second_workload and args.second_workload != args.workload:
        del views
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        m2 = second_context_length(args.second_workload, dev, args, timer)
        result["second_workload"] = m2
        log(f"{m2['config']['workload']}: {m2['value'] / 1e9:.3f} G tokens/s, stream "
            f"{m2['roofline']['frac']:.3f} of peak, step {m2['step_roofline']['frac']:.3f}")
    # numerics check of the timed outputs against the oracle (CPU baseline leg)
    if not args.no_cpu_baseline:
        cb = cpu_baseline(cfg, 0)
        if cb is not None:
            base, res = cb
            result["cpu_baseline"] = base
            ada.decode(geom, cache, L["cb8"], L["cb4"], L["q"], cfg.sigma, out, lse,
                       num_splits=args.splits, ws=ws)
            torch.cuda.synchronize()
            result["parity_out_max_abs"] = float(np.abs(out.cpu().double().numpy() - res["out"]).max())
    print(json.dumps(result))


if __name__ == "__main__":
    main()
