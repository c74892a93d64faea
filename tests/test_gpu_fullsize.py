"""Full-size parity for the large workloads (GPU).

The whole workload runs on the GPU exactly as the benchmark runs it: encode,
pack into a (permuted) pool, decode with the default split count.  The
oracle then builds its own cache from the same synthetic inputs for a sample
of sequences -- a sequence's pages, and so its outputs, depend on no other
sequence -- and the two are compared:
  * radii and codes bit-exact;
  * every page of every sampled row bit-exact, with its metadata, page count
    and tier counts (pages are found through each side's own page table);
  * outputs max-abs <= 1e-2 and lse within 1e-3 * max(|lse|, 1).
The GPU pool itself must be exactly tiled by the pages of every row.
"""
from __future__ import annotations

import os

import numpy as np
import pytest
import torch

import compressed_kv_attention_amd as ada
import oracle
import synth
from gpu_util import flush, u16

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2
NTHREADS = max(1, min(os.cpu_count() or 1, 16))


def _stored_bytes(cfg, lens, bp, extra_tokens=0):
    H, D = cfg.num_kv_heads, cfg.head_dim
    total = 0
    for s, T in enumerate(lens):
        for T_call in ([int(T)] + ([extra_tokens] if extra_tokens else [])):
            n = [(int(bp[s][k]) * T_call + 5000) // 10000 for k in range(3)]
            cnt = [n[0], n[1] - n[0], n[2] - n[1]]
            total += H * sum((c + 15) // 16 * ada.page_bytes(D, k) for k, c in enumerate(cnt))
    return total


def _gpu_encode(geom, keys, cb8, cb4):
    n, H, D = keys.shape
    r = torch.empty((n, H), dtype=torch.float16, device="cuda")
    c8 = torch.empty((n, H, D // 8), dtype=torch.uint8, device="cuda")
    c4 = torch.empty((n, H, D // 16), dtype=torch.uint8, device="cuda")
    ada.encode(geom, keys, cb8, cb4, r, c8, c4)
    return r, c8, c4


def _check_codes(label, g_r, g_c8, g_c4, keys_cpu, cb8, cb4):
    """GPU encode outputs of a token sample against the oracle's: bit-exact
    (the kernel's binary32 filter only skips the double scan where its bound
    proves the winner, so its codes are the defining argmin)."""
    rr, rc8, rc4 = oracle.encode(keys_cpu, cb8, cb4, nthreads=NTHREADS)
    assert np.array_equal(u16(g_r), rr), f"{label}: radius differs"
    g8, g4 = g_c8.cpu().numpy(), g_c4.cpu().numpy()
    bad = np.nonzero((g8 != rc8).any((1, 2)) | (g4 != rc4).any((1, 2)))[0]
    assert len(bad) == 0, f"{label}: codes of {len(bad)} tokens differ (first {bad[:5].tolist()})"
    flush(f"[{label}] codes of {len(g8)} tokens bit-exact")
    return rr, rc8, rc4


def _check_pool_tiling(label, dc, geom):
    """The GPU pool is exactly tiled by the pages of all rows: no gap, no
    overlap, ending at the arena cursor."""
    npg = dc.num_pages.cpu().numpy()
    pt = dc.page_table.cpu().numpy().view(np.uint32)
    pm = dc.page_meta.cpu().numpy()
    offs, sizes = [], []
    for r in range(len(npg)):
        n = int(npg[r])
        offs.append(pt[r, :n].astype(np.int64) * 128)
        sizes.append(np.array([ada.page_bytes(geom.head_dim, int(m) & 3) for m in pm[r, :n]], np.int64))
    offs, sizes = np.concatenate(offs), np.concatenate(sizes)
    order = np.argsort(offs)
    o, z = offs[order], sizes[order]
    assert o[0] == 0 and np.array_equal(o[1:], (o + z)[:-1]), f"{label}: pool not tiled"
    assert int(o[-1] + z[-1]) == int(dc.cursor[0]) * 128
    flush(f"[{label}] pool of {len(o)} pages exactly tiled")


def _compare_rows(label, dc, arena_gpu, hc, seqs, H, D):
    """Pages, metadata and counts of the sampled rows, bit-exact."""
    npg = dc.num_pages.cpu().numpy()
    pt = dc.page_table.cpu().numpy().view(np.uint32)
    pm = dc.page_meta.cpu().numpy()
    tt = dc.tier_tokens.cpu().numpy()
    for i, s in enumerate(seqs):
        for h in range(H):
            rg, ro = s * H + h, i * H + h
            n = int(hc.num_pages[ro])
            assert int(npg[rg]) == n, f"{label}: row ({s},{h}) page count"
            assert np.array_equal(pm[rg, :n], hc.page_meta[ro, :n]), f"{label}: row ({s},{h}) metadata"
            assert np.array_equal(tt[rg], hc.tier_tokens[ro]), f"{label}: row ({s},{h}) tier counts"
            if n == 0:
                continue
            sizes = [ada.page_bytes(D, int(m) & 3) for m in pm[rg, :n]]
            g = torch.cat([arena_gpu[int(pt[rg, p]) * 128: int(pt[rg, p]) * 128 + sizes[p]]
                           for p in range(n)]).cpu().numpy()
            o = np.concatenate([hc.arena[int(hc.page_table[ro, p]) * 128: int(hc.page_table[ro, p]) * 128 + sizes[p]]
                                for p in range(n)])
            if not np.array_equal(g, o):
                first = int(np.nonzero(g != o)[0][0])
                page = int(np.searchsorted(np.cumsum(sizes), first, side="right"))
                raise AssertionError(f"{label}: row ({s},{h}) page {page} bytes differ")
    flush(f"[{label}] pages of {len(seqs) * H} sampled rows bit-exact")


def _check_outputs(label, out, lse, ref, seqs):
    o = out[seqs].cpu().double().numpy()
    err = np.abs(o - ref["out"]).max()
    assert err <= OUT_TOL, f"{label}: out max-abs {err:.3g}"
    l = lse[seqs].cpu().double().numpy()
    assert (np.abs(l - ref["lse"]) <= 1e-3 * np.maximum(np.abs(ref["lse"]), 1.0)).all(), f"{label}: lse"
    flush(f"[{label}] outputs of {len(seqs)} sampled sequences: max-abs {err:.2e}")


def _run(number, layer, seqs, append=0):
    cfg = synth.WORKLOADS[number]
    label = f"workload {number} layer {layer}"
    flush(f"[{label}] building inputs on the GPU")
    H, D, S = cfg.num_kv_heads, cfg.head_dim, cfg.num_seqs
    geom = ada.Geom(D, cfg.num_q_heads, H)
    lens = synth.seq_lens(cfg)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    bp = synth.tier_mix(cfg)
    keys = synth.keys(cfg, layer, N, "cuda")
    vals = synth.values(cfg, layer, N, "cuda")
    scores = synth.scores(cfg, layer, N)
    q = synth.queries(cfg, layer, "cuda")
    cb8, cb4 = synth.codebooks(cfg, layer)
    cb8d, cb4d = cb8.cuda(), cb4.cuda()

    # --- the GPU path at full size ------------------------------------------
    flush(f"[{label}] GPU encode + pack of {N} tokens x {H} heads")
    r, c8, c4 = _gpu_encode(geom, keys, cb8d, cb4d)
    maxp = int(max(lens)) // 16 + 4 + (append // 16 + 4 if append else 0)
    dc = ada.Cache(geom, S, maxp, _stored_bytes(cfg, lens, bp, append))
    n_pages = ada.pack_num_pages(geom, cu, bp)
    ada.rdr_pack(geom, dc, cu, bp, keys, vals, r, c8, c4, scores.cuda(),
                 place_perm=synth.place_perm(cfg, layer, n_pages))
    if append:
        acu = synth.cu_tokens(np.full(S, append, np.int64))
        ak = synth.keys(cfg, layer, S * append, "cuda", stream="k-append")
        av = synth.values(cfg, layer, S * append, "cuda", stream="v-append")
        asc = synth.scores(cfg, layer, S * append, stream="score-append")
        ar, ac8, ac4 = _gpu_encode(geom, ak, cb8d, cb4d)
        an = ada.pack_num_pages(geom, acu, bp)
        ada.rdr_pack(geom, dc, acu, bp, ak, av, ar, ac8, ac4, asc.cuda(),
                     place_perm=synth.place_perm(cfg, layer, an, stream="place-append"),
                     pos_base=lens.astype(np.int64))
    out = torch.full((S, cfg.num_q_heads, D), float("nan"), device="cuda")
    lse = torch.full((S, cfg.num_q_heads), float("nan"), device="cuda")
    ada.decode(geom, dc, cb8d, cb4d, q, cfg.sigma, out, lse)
    torch.cuda.synchronize()
    _check_pool_tiling(label, dc, geom)

    # --- the oracle on the sampled sequences ----------------------------------
    sl = [slice(int(cu[s]), int(cu[s + 1])) for s in seqs]
    k_s = torch.cat([keys[x] for x in sl]).cpu()
    v_s = torch.cat([vals[x] for x in sl]).cpu()
    sc_s = torch.cat([scores[x] for x in sl])
    flush(f"[{label}] oracle encode of {len(k_s)} tokens x {H} heads ({NTHREADS} threads)")
    rr, rc8, rc4 = _check_codes(label, torch.cat([r[x] for x in sl]), torch.cat([c8[x] for x in sl]),
                                torch.cat([c4[x] for x in sl]), k_s, cb8, cb4)
    lens_s = lens[seqs]
    cu_s = synth.cu_tokens(lens_s)
    bp_s = bp[seqs]
    hc = oracle.HostCache(D, H, len(seqs), maxp, _stored_bytes(cfg, lens_s, bp_s, append) + 4096,
                          slot_tokens=False)
    assert oracle.pack(hc, cu_s, bp_s, k_s, v_s, rr, rc8, rc4, sc_s) == 0
    if append:
        ak_s = torch.cat([ak[s * append:(s + 1) * append] for s in seqs]).cpu()
        av_s = torch.cat([av[s * append:(s + 1) * append] for s in seqs]).cpu()
        asc_s = torch.cat([asc[s * append:(s + 1) * append] for s in seqs])
        arr, arc8, arc4 = _check_codes(label + " append", torch.cat([ar[s * append:(s + 1) * append] for s in seqs]),
                                       torch.cat([ac8[s * append:(s + 1) * append] for s in seqs]),
                                       torch.cat([ac4[s * append:(s + 1) * append] for s in seqs]),
                                       ak_s, cb8, cb4)
        acu_s = synth.cu_tokens(np.full(len(seqs), append, np.int64))
        assert oracle.pack(hc, acu_s, bp_s, ak_s, av_s, arr, arc8, arc4, asc_s,
                           pos_base=lens_s.astype(np.int64)) == 0
    _compare_rows(label, dc, dc.arena, hc, seqs, H, D)
    flush(f"[{label}] oracle decode of {len(seqs)} sequences")
    ref = oracle.decode(hc, cb8, cb4, q[seqs].cpu(), cfg.sigma, nthreads=NTHREADS)
    _check_outputs(label, out, lse, ref, seqs)


def test_workload3_batch4_t128k_permuted_pool():
    _run(3, 0, [0, 3])


def test_workload4_ragged64_budgets():
    lens = synth.seq_lens(synth.WORKLOADS[4])
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 17})
    _run(4, 0, seqs)


def test_workload5_one_layer_t128k_with_append():
    _run(5, 7, [2, 5], append=synth.WORKLOADS[5].append_tokens)


def test_workload6_qwen_shape_gqa5_t32k():
    _run(6, 0, [0])


def test_workload7_gpt_oss_shape_gqa8_d64_t32k():
    _run(7, 0, [0])


def _run_solver(number, layer, seqs):
    """The append path with the budget solver at full size: GPU encode, code
    error, solve under each sequence's byte budget, tier counts, tier-given
    pack into a permuted pool, decode; then the oracle on the sampled
    sequences (each sequence's solve depends on no other)."""
    cfg = synth.WORKLOADS[number]
    label = f"workload {number} budget solver"
    H, D, S = cfg.num_kv_heads, cfg.head_dim, cfg.num_seqs
    geom = ada.Geom(D, cfg.num_q_heads, H)
    lens = synth.seq_lens(cfg)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    budgets = synth.budget_bytes(cfg, lens)
    flush(f"[{label}] GPU encode, code error and solve of {N} tokens x {H} heads")
    keys = synth.keys(cfg, layer, N, "cuda")
    vals = synth.values(cfg, layer, N, "cuda")
    scores = synth.scores(cfg, layer, N)
    q = synth.queries(cfg, layer, "cuda")
    cb8, cb4 = synth.codebooks(cfg, layer)
    cb8d, cb4d = cb8.cuda(), cb4.cuda()
    r, c8, c4 = _gpu_encode(geom, keys, cb8d, cb4d)
    e8 = torch.empty((N, H), device="cuda")
    e4 = torch.empty((N, H), device="cuda")
    ada.code_error(geom, keys, cb8d, cb4d, c8, c4, e8, e4)
    tiers = torch.empty((N, H), dtype=torch.uint8, device="cuda")
    ada.rdr_solve(geom, cu, budgets, r, e8, e4, scores.cuda(), tiers)
    counts = ada.tier_counts(geom, cu, tiers)
    n_pages = ada.pack_tiers_num_pages(geom, counts)
    per_seq = np.zeros(S, np.int64)
    for s in range(S):
        for row in counts[s * H:(s + 1) * H]:
            per_seq[s] += sum(ada.page_bytes(D, k) * -(-int(c) // 16) for k, c in enumerate(row))
    assert (per_seq <= budgets).all(), f"{label}: a sequence exceeds its budget"
    maxp = int(max(lens)) // 16 + 4
    dc = ada.Cache(geom, S, maxp, int(per_seq.sum()))
    ada.rdr_pack_tiers(geom, dc, cu, counts, tiers, keys, vals, r, c8, c4,
                       place_perm=synth.place_perm(cfg, layer, n_pages))
    out = torch.full((S, cfg.num_q_heads, D), float("nan"), device="cuda")
    lse = torch.full((S, cfg.num_q_heads), float("nan"), device="cuda")
    ada.decode(geom, dc, cb8d, cb4d, q, cfg.sigma, out, lse)
    torch.cuda.synchronize()
    _check_pool_tiling(label, dc, geom)
    mix = np.bincount(tiers.cpu().numpy().ravel(), minlength=4) / (N * H)
    flush(f"[{label}] tier mix {np.round(mix, 3)}, stored {per_seq.sum() / 1e6:.1f} MB")

    sl = [slice(int(cu[s]), int(cu[s + 1])) for s in seqs]
    k_s = torch.cat([keys[x] for x in sl]).cpu()
    v_s = torch.cat([vals[x] for x in sl]).cpu()
    sc_s = torch.cat([scores[x] for x in sl]).numpy()
    g_r = torch.cat([r[x] for x in sl])
    g_c8 = torch.cat([c8[x] for x in sl])
    g_c4 = torch.cat([c4[x] for x in sl])
    flush(f"[{label}] oracle on {len(k_s)} tokens x {H} heads ({NTHREADS} threads)")
    _check_codes(label, g_r, g_c8, g_c4, k_s, cb8, cb4)
    # downstream of the codes the oracle takes the GPU's (equal, as checked)
    gr, gc8, gc4 = u16(g_r), g_c8.cpu().numpy(), g_c4.cpu().numpy()
    re8, re4 = oracle.code_error(k_s, cb8, cb4, gc8, gc4)
    assert np.array_equal(torch.cat([e8[x] for x in sl]).cpu().numpy(), re8), f"{label}: err8"
    assert np.array_equal(torch.cat([e4[x] for x in sl]).cpu().numpy(), re4), f"{label}: err4"
    lens_s = lens[seqs]
    cu_s = synth.cu_tokens(lens_s)
    rt = oracle.rdr_solve(D, cu_s, budgets[seqs], gr, re8, re4, sc_s)
    assert np.array_equal(torch.cat([tiers[x] for x in sl]).cpu().numpy(), rt), f"{label}: tiers"
    flush(f"[{label}] code errors and tiers of the sampled sequences bit-exact")
    hc = oracle.HostCache(D, H, len(seqs), maxp, int(per_seq[seqs].sum()) + 4096, slot_tokens=False)
    assert oracle.pack_tiers(hc, cu_s, rt, k_s, v_s, gr, gc8, gc4) == 0
    _compare_rows(label, dc, dc.arena, hc, seqs, H, D)
    ref = oracle.decode(hc, cb8, cb4, q[seqs].cpu(), cfg.sigma, nthreads=NTHREADS)
    _check_outputs(label, out, lse, ref, seqs)


def test_workload4_ragged64_with_budget_solver():
    lens = synth.seq_lens(synth.WORKLOADS[4])
    seqs = sorted({int(np.argmin(lens)), int(np.argmax(lens)), 17})
    _run_solver(4, 0, seqs)


def test_workload2_budget_solver_60pct():
    _run_solver(2, 0, [0])


def test_single_row_gqa8_d128_t128k_lds_bound_splits():
    """One (sequence, kv-head) row of 131072 tokens with 8 query heads at
    D = 128: the LUT fills most of LDS, so the default split count is set by
    the page-table room; every head of the row against the oracle."""
    from helpers import make_case, oracle_cache, small_workload
    cfg = small_workload(D=128, Hq=8, Hkv=1, S=1, T=131072, mix=(1000, 5000, 8000), seed=300,
                         samples=4096, iters=4)
    case = make_case(cfg)
    flush("[gqa8 t128k] oracle encode + pack")
    hc, _ = oracle_cache(case, slot_tokens=False)
    geom = ada.Geom(128, 8, 1)
    from gpu_util import upload_cache, to_dev
    dc = upload_cache(hc, geom)
    ns = ada.decode_default_splits(geom, 1, hc.maxp)
    flush(f"[gqa8 t128k] {int(hc.num_pages[0])} pages, {ns} splits")
    out = torch.full((1, 8, 128), float("nan"), device="cuda")
    lse = torch.full((1, 8), float("nan"), device="cuda")
    ada.decode(geom, dc, to_dev(case["cb8"]), to_dev(case["cb4"]), to_dev(case["q"]), cfg.sigma, out, lse)
    torch.cuda.synchronize()
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, nthreads=NTHREADS)
    _check_outputs("gqa8 t128k", out, lse, ref, [0])


# ---- every sequence, with the GPU's encode outputs fed to the oracle ---------
# Pages, tables and outputs are compared for every sequence of a workload.
# The oracle's pack and decode take the GPU's radii and codes (checked bit
# for bit against the oracle's own encode on a seeded token sample first), as
# both packs must see the same encode outputs; oracle encode of every token
# of the large workloads would take minutes of CPU time.

def _host_tables(dc):
    return dict(npg=dc.num_pages.cpu().numpy(), pt=dc.page_table.cpu().numpy().view(np.uint32),
                pm=dc.page_meta.cpu().numpy(), tt=dc.tier_tokens.cpu().numpy())


def _tier_pages(units, pt_row, pm_row, D):
    """The row's pages of each tier in page order, as [n][bytes] arrays."""
    out = []
    for k in range(3):
        sel = (pm_row & 3) == k
        u = ada.page_bytes(D, k) // 128
        idx = pt_row[sel].astype(np.int64)[:, None] + np.arange(u)[None, :]
        out.append(units[idx].reshape(len(idx), -1))
    return out


def _compare_rows_all(label, arena_g, tab, hc, pairs, D):
    """Bit-exact pages, metadata and counts for (GPU row, oracle row) pairs,
    each side's pages found through its own page table."""
    A = arena_g[: len(arena_g) // 128 * 128].reshape(-1, 128)
    B = hc.arena[: len(hc.arena) // 128 * 128].reshape(-1, 128)
    for rg, ro in pairs:
        n = int(hc.num_pages[ro])
        assert int(tab["npg"][rg]) == n, f"{label}: row {rg} page count"
        assert np.array_equal(tab["pm"][rg, :n], hc.page_meta[ro, :n]), f"{label}: row {rg} metadata"
        assert np.array_equal(tab["tt"][rg], hc.tier_tokens[ro]), f"{label}: row {rg} tier counts"
        ga = _tier_pages(A, tab["pt"][rg, :n], tab["pm"][rg, :n], D)
        oa = _tier_pages(B, hc.page_table[ro, :n], hc.page_meta[ro, :n], D)
        for k in range(3):
            assert np.array_equal(ga[k], oa[k]), f"{label}: row {rg} tier-{k} page bytes differ"


def _sample_codes(label, keys, r, c8, c4, cb8, cb4, n, seed):
    N = keys.shape[0]
    idx = np.sort(np.random.default_rng(seed).choice(N, min(n, N), replace=False))
    it = torch.from_numpy(idx).cuda()
    _check_codes(label + " token sample", r[it], c8[it], c4[it], keys[it].cpu(), cb8, cb4)


def _oracle_chunk(label, cfg, layer, seqs, lens, bp, cu, keys, vals, scores, g_r, g_c8, g_c4, maxp):
    """Oracle pack of sequences seqs (contiguous) from the GPU's codes."""
    H, D = cfg.num_kv_heads, cfg.head_dim
    a, b = int(cu[seqs[0]]), int(cu[seqs[-1] + 1])
    lens_s, bp_s = lens[seqs], bp[seqs]
    hc = oracle.HostCache(D, H, len(seqs), maxp, _stored_bytes(cfg, lens_s, bp_s) + 4096, slot_tokens=False)
    rc = oracle.pack(hc, synth.cu_tokens(lens_s), bp_s, keys[a:b].cpu(), vals[a:b].cpu(), g_r[a:b], g_c8[a:b],
                     g_c4[a:b], scores[a:b])
    assert rc == 0, f"{label}: oracle pack {rc}"
    return hc


def _run_all_seqs(number, layer, chunk, logits_seq=None):
    cfg = synth.WORKLOADS[number]
    label = f"workload {number} all sequences"
    H, D, S, Hq = cfg.num_kv_heads, cfg.head_dim, cfg.num_seqs, cfg.num_q_heads
    geom = ada.Geom(D, Hq, H)
    lens = synth.seq_lens(cfg)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    bp = synth.tier_mix(cfg)
    flush(f"[{label}] GPU encode + pack of {N} tokens x {H} heads, decode")
    keys = synth.keys(cfg, layer, N, "cuda")
    vals = synth.values(cfg, layer, N, "cuda")
    scores = synth.scores(cfg, layer, N)
    q = synth.queries(cfg, layer, "cuda")
    cb8, cb4 = synth.codebooks(cfg, layer)
    cb8d, cb4d = cb8.cuda(), cb4.cuda()
    r, c8, c4 = _gpu_encode(geom, keys, cb8d, cb4d)
    maxp = int(max(lens)) // 16 + 4
    dc = ada.Cache(geom, S, maxp, _stored_bytes(cfg, lens, bp))
    n_pages = ada.pack_num_pages(geom, cu, bp)
    ada.rdr_pack(geom, dc, cu, bp, keys, vals, r, c8, c4, scores.cuda(),
                 place_perm=synth.place_perm(cfg, layer, n_pages))
    out = torch.full((S, Hq, D), float("nan"), device="cuda")
    lse = torch.full((S, Hq), float("nan"), device="cuda")
    lg = torch.full((S, Hq, maxp * 16), float("nan"), device="cuda") if logits_seq is not None else None
    ada.decode(geom, dc, cb8d, cb4d, q, cfg.sigma, out, lse, logits=lg)
    torch.cuda.synchronize()
    _check_pool_tiling(label, dc, geom)
    _sample_codes(label, keys, r, c8, c4, cb8, cb4, 4096, 100 + number)
    arena_g = dc.arena.cpu().numpy()
    tab = _host_tables(dc)
    g_r, g_c8, g_c4 = u16(r), c8.cpu().numpy(), c4.cpu().numpy()
    del r, c8, c4
    worst = 0.0
    for s0 in range(0, S, chunk):
        seqs = list(range(s0, min(S, s0 + chunk)))
        hc = _oracle_chunk(label, cfg, layer, seqs, lens, bp, cu, keys, vals, scores, g_r, g_c8, g_c4, maxp)
        _compare_rows_all(label, arena_g, tab, hc, [(s * H + h, i * H + h) for i, s in enumerate(seqs)
                                                    for h in range(H)], D)
        want_lg = logits_seq is not None and logits_seq in seqs
        ref = oracle.decode(hc, cb8, cb4, q[seqs].cpu(), cfg.sigma, nthreads=NTHREADS, logits=want_lg)
        o = out[seqs].cpu().double().numpy()
        err = float(np.abs(o - ref["out"]).max())
        assert err <= OUT_TOL, f"{label}: sequences {seqs[0]}..{seqs[-1]} out max-abs {err:.3g}"
        ls = lse[seqs].cpu().double().numpy()
        assert (np.abs(ls - ref["lse"]) <= 1e-3 * np.maximum(np.abs(ref["lse"]), 1.0)).all(), f"{label}: lse"
        worst = max(worst, err)
        if want_lg:
            from gpu_util import logit_tol_ok
            i = seqs.index(logits_seq)
            ok, rel = logit_tol_ok(lg[logits_seq].cpu().double().numpy(), ref["logits"][i])
            assert ok, f"{label}: sequence {logits_seq} logits rel err {rel:.3g}"
            flush(f"[{label}] logits of sequence {logits_seq} (all {Hq} heads, every retained slot): "
                  f"max rel {rel:.2e}")
        flush(f"[{label}] sequences {seqs[0]}..{seqs[-1]}: pages of {len(seqs) * H} rows bit-exact, "
              f"out max-abs {err:.2e}")
    flush(f"[{label}] all {S} sequences: out max-abs {worst:.2e}")


def test_workload3_all_sequences_and_full_logits():
    """Every sequence of the 4 x 131072 permuted pool, and the logits of every
    retained slot of one sequence at full size."""
    _run_all_seqs(3, 0, chunk=2, logits_seq=1)


def test_workload4_all_64_sequences():
    """Every one of the 64 ragged sequences: pages bit-exact and outputs."""
    _run_all_seqs(4, 0, chunk=16)


def test_workload5_four_layers_back_to_back():
    """Several layers of the 32-layer workload, each with its own keys,
    values, queries, codebooks and cache, decoded back to back on one stream
    into separate outputs (the order the benchmark times them in); each
    layer's outputs for a sampled sequence against the oracle."""
    cfg = synth.WORKLOADS[5]
    H, D, S, Hq = cfg.num_kv_heads, cfg.head_dim, cfg.num_seqs, cfg.num_q_heads
    geom = ada.Geom(D, Hq, H)
    lens = synth.seq_lens(cfg)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    bp = synth.tier_mix(cfg)
    maxp = int(max(lens)) // 16 + 4
    layers = [0, 11, 22, 31]
    built = []
    for layer in layers:
        label = f"workload 5 layer {layer}"
        flush(f"[{label}] GPU encode + pack of {N} tokens x {H} heads")
        keys = synth.keys(cfg, layer, N, "cuda")
        vals = synth.values(cfg, layer, N, "cuda")
        scores = synth.scores(cfg, layer, N)
        cb8, cb4 = synth.codebooks(cfg, layer)
        cb8d, cb4d = cb8.cuda(), cb4.cuda()
        r, c8, c4 = _gpu_encode(geom, keys, cb8d, cb4d)
        dc = ada.Cache(geom, S, maxp, _stored_bytes(cfg, lens, bp))
        ada.rdr_pack(geom, dc, cu, bp, keys, vals, r, c8, c4, scores.cuda(),
                     place_perm=synth.place_perm(cfg, layer, ada.pack_num_pages(geom, cu, bp)))
        s = (3 * layer + 1) % S  # the layer's sampled sequence
        a, b = int(cu[s]), int(cu[s + 1])
        _sample_codes(label, keys[a:b], r[a:b], c8[a:b], c4[a:b], cb8, cb4, 1024, layer)
        torch.cuda.synchronize()
        built.append(dict(layer=layer, s=s, dc=dc, cb8=cb8, cb4=cb4, cb8d=cb8d, cb4d=cb4d,
                          q=synth.queries(cfg, layer, "cuda"), k=keys[a:b].cpu(), v=vals[a:b].cpu(),
                          sc=scores[a:b], r=u16(r[a:b]), c8=c8[a:b].cpu().numpy(),
                          c4=c4[a:b].cpu().numpy()))
        del keys, vals, r, c8, c4
    outs = [torch.full((S, Hq, D), float("nan"), device="cuda") for _ in layers]
    lses = [torch.full((S, Hq), float("nan"), device="cuda") for _ in layers]
    ws = torch.zeros(ada.decode_workspace_size(geom, S, maxp, 0), dtype=torch.uint8, device="cuda")
    flush(f"[workload 5] {len(layers)} layers decoded back to back on one stream")
    for B, o, l in zip(built, outs, lses):
        ada.decode(geom, B["dc"], B["cb8d"], B["cb4d"], B["q"], cfg.sigma, o, l, ws=ws)
    torch.cuda.synchronize()
    for B, o, l in zip(built, outs, lses):
        label = f"workload 5 layer {B['layer']}"
        s = B["s"]
        hc = oracle.HostCache(D, H, 1, maxp, _stored_bytes(cfg, lens[[s]], bp[[s]]) + 4096, slot_tokens=False)
        assert oracle.pack(hc, synth.cu_tokens(lens[[s]]), bp[[s]], B["k"], B["v"], B["r"], B["c8"], B["c4"],
                           B["sc"]) == 0
        _compare_rows_all(label, B["dc"].arena.cpu().numpy(), _host_tables(B["dc"]), hc,
                          [(s * H + h, h) for h in range(H)], D)
        ref = oracle.decode(hc, B["cb8"], B["cb4"], B["q"][[s]].cpu(), cfg.sigma, nthreads=NTHREADS)
        _check_outputs(label, o, l, ref, [s])
