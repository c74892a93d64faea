"""GPU parity of the decode-step append (ada_append) through the C ABI.

Bars: tiers given to the new states, every row's pages (found through each
side's own page table: rows race for the arena cursor, so offsets differ),
metadata, page counts, tier counts, slot positions and the final cursor are
bit-exact against the oracle after many steps; the solver's threshold output
bit-exact; decode after the appends within the decode bars; a step captured
in a graph and replayed gives what eager steps give."""
import numpy as np
import pytest
import torch

import compressed_kv_attention_amd as ada
import oracle
import synth
from gpu_util import decode_outputs, flush, geom_of, to_dev, upload_cache
from helpers import make_case, small_workload

pytestmark = pytest.mark.gpu
OUT_TOL = 1e-2


def _base(cfg, lens, frac, maxp_extra):
    """An oracle-built cache from the budget solver, plus the thresholds."""
    case = make_case(cfg, lens=lens)
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"], nthreads=8)
    e8, e4 = oracle.code_error(case["keys"], case["cb8"], case["cb4"], c8, c4)
    budgets = synth.budget_bytes(cfg, lens) * frac // 100
    tiers, th = oracle.rdr_solve(cfg.head_dim, case["cu"], budgets, r, e8, e4, case["scores"].numpy(),
                                 with_threshold=True)
    maxp = max(lens) // 16 + 4 + maxp_extra
    arena = int(sum(lens) * cfg.num_kv_heads * 512 + 3 * len(lens) * cfg.num_kv_heads * 8192
                + maxp_extra * len(lens) * cfg.num_kv_heads * 8192)
    hc = oracle.HostCache(cfg.head_dim, cfg.num_kv_heads, len(lens), maxp, arena)
    assert oracle.pack_tiers(hc, case["cu"], tiers, case["keys"], case["values"], r, c8, c4,
                             pos_base=np.zeros(len(lens), np.int64)) == 0
    return case, hc, th, (r, e8, e4, budgets)


def _upload(hc, geom):
    dc = upload_cache(hc, geom, slot_tokens=True)
    dc.slot_token.copy_(torch.from_numpy(hc.slot_token))
    return dc


def _compare(dc, hc, label):
    npg = dc.num_pages.cpu().numpy()
    pt = dc.page_table.cpu().numpy().view(np.uint32)
    pm = dc.page_meta.cpu().numpy()
    sl = dc.slot_token.cpu().numpy()
    ar = dc.arena.cpu().numpy()
    assert np.array_equal(npg[: len(hc.num_pages)], hc.num_pages), f"{label}: page counts"
    assert np.array_equal(dc.tier_tokens.cpu().numpy()[: len(hc.num_pages)], hc.tier_tokens), f"{label}: tiers"
    for row in range(len(hc.num_pages)):
        for p in range(int(hc.num_pages[row])):
            assert pm[row, p] == hc.page_meta[row, p], f"{label}: row {row} page {p} meta"
            n = oracle.page_bytes(hc.D, int(pm[row, p]) & 3)
            g = ar[int(pt[row, p]) * 128: int(pt[row, p]) * 128 + n]
            assert np.array_equal(g, hc.page(row, p)), f"{label}: row {row} page {p} bytes"
            assert np.array_equal(sl[row, p], hc.slot_token[row, p]), f"{label}: row {row} page {p} slots"


def _new_tokens(cfg, step, S):
    k = synth.keys(cfg, 0, S, stream=f"k-step{step}").contiguous()
    v = synth.values(cfg, 0, S, stream=f"v-step{step}").contiguous()
    sc = synth.scores(cfg, 0, S, stream=f"s-step{step}").contiguous()
    return k, v, sc


@pytest.mark.parametrize("D,frac", [(128, 60), (64, 45)])
def test_append_steps_bit_exact_then_decode(D, frac):
    cfg = small_workload(D=D, Hq=8, Hkv=2, S=3, T=300, seed=200 + D)
    lens = [300, 180, 41]
    case, hc, th, _ = _base(cfg, lens, frac, 4)
    geom = geom_of(cfg)
    dc = _upload(hc, geom)
    state = ada.AppendState(geom, dc)
    open_page = np.zeros((3 * 2, 3), np.int32)
    cb8, cb4 = to_dev(case["cb8"]), to_dev(case["cb4"])
    th_d = to_dev(th)
    S = len(lens)
    tiers_all = []
    for step in range(40):
        k, v, sc = _new_tokens(cfg, step, S)
        pos = np.array(lens, np.int64) + step
        tg = torch.full((S, 2), 77, dtype=torch.uint8, device="cuda")
        ada.append(geom, dc, state, cb8, cb4, to_dev(k), to_dev(v), to_dev(sc), th_d, to_dev(pos), tiers=tg)
        to, st = oracle.append(hc, k, v, sc.numpy(), case["cb8"], case["cb4"], th, pos, open_page)
        assert st == 0
        assert np.array_equal(tg.cpu().numpy(), to), f"step {step}: tiers"
        tiers_all.append(to)
    flush(f"[append] D={D}: 40 steps, tier mix {np.bincount(np.concatenate(tiers_all).ravel(), minlength=4)}")
    assert state.pull() == 0
    assert int(dc.cursor[0]) == int(hc.cursor[0])
    assert np.array_equal(state.buf[256:256 + 6 * 3 * 4].cpu().numpy().view(np.int32).reshape(6, 3), open_page)
    _compare(dc, hc, f"append D={D}")
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, nthreads=8)
    out, lse, _ = decode_outputs(geom, dc, to_dev(case["q"]), with_logits=False)
    ada.decode(geom, dc, cb8, cb4, to_dev(case["q"]), cfg.sigma, out, lse)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().double().numpy() - ref["out"]).max() <= OUT_TOL


def test_solver_threshold_output_bit_exact():
    cfg = small_workload(D=128, Hq=4, Hkv=2, S=4, T=500, seed=210)
    lens = [500, 0, 230, 64]
    case = make_case(cfg, lens=lens)
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"], nthreads=8)
    e8, e4 = oracle.code_error(case["keys"], case["cb8"], case["cb4"], c8, c4)
    geom = geom_of(cfg)
    for frac in (0, 30, 70, 120):
        budgets = synth.budget_bytes(cfg, lens) * frac // 100
        tiers, th = oracle.rdr_solve(128, case["cu"], budgets, r, e8, e4, case["scores"].numpy(),
                                     with_threshold=True)
        gt = torch.empty((case["N"], 2), dtype=torch.uint8, device="cuda")
        gth = torch.full((4,), float("nan"), device="cuda")
        ada.rdr_solve(geom, case["cu"], budgets, to_dev(r), to_dev(e8), to_dev(e4), to_dev(case["scores"]), gt,
                      threshold=gth)
        torch.cuda.synchronize()
        assert np.array_equal(gt.cpu().numpy(), tiers)
        assert np.array_equal(gth.cpu().numpy(), th), (frac, gth.cpu().numpy(), th)


def test_append_capacity_status_bits():
    cfg = small_workload(D=64, Hq=2, Hkv=1, S=1, T=16, seed=220)
    geom = geom_of(cfg)
    case = make_case(cfg, lens=[16])
    cb8, cb4 = to_dev(case["cb8"]), to_dev(case["cb4"])
    neg = torch.full((1,), float("-inf"), device="cuda")  # every state stays fp16
    # page table of 2 pages: the 33rd token has nowhere to go
    dc = ada.Cache(geom, 1, 2, 1 << 20, slot_tokens=True)
    state = ada.AppendState(geom, dc)
    for step in range(34):
        k, v, sc = _new_tokens(cfg, step, 1)
        ada.append(geom, dc, state, cb8, cb4, to_dev(k), to_dev(v), to_dev(sc), neg,
                   torch.tensor([step], dtype=torch.int64, device="cuda"))
    assert state.pull() == 1 and int(dc.num_pages[0]) == 2 and int(dc.tier_tokens[0, 0]) == 32
    # arena of exactly two fp16 pages (32 units each at D = 64)
    dc = ada.Cache(geom, 1, 8, 2 * 4096, slot_tokens=True)
    state = ada.AppendState(geom, dc)
    for step in range(40):
        k, v, sc = _new_tokens(cfg, step, 1)
        ada.append(geom, dc, state, cb8, cb4, to_dev(k), to_dev(v), to_dev(sc), neg,
                   torch.tensor([step], dtype=torch.int64, device="cuda"))
    assert state.pull() == 2 and int(dc.num_pages[0]) == 2 and int(dc.cursor[0]) == 64


def test_append_step_in_a_graph_equals_eager():
    cfg = small_workload(D=128, Hq=8, Hkv=2, S=2, T=100, seed=230)
    lens = [100, 37]
    case, hc, th, _ = _base(cfg, lens, 55, 2)
    geom = geom_of(cfg)
    cb8, cb4 = to_dev(case["cb8"]), to_dev(case["cb4"])
    th_d = to_dev(th)
    eager = _upload(hc, geom)
    es = ada.AppendState(geom, eager)
    graphed = _upload(hc, geom)
    gs = ada.AppendState(geom, graphed)
    kb = torch.empty((2, 2, 128), dtype=torch.float16, device="cuda")
    vb = torch.empty((2, 2, 128), dtype=torch.bfloat16, device="cuda")
    sb = torch.empty((2, 2), device="cuda")
    pb = torch.empty(2, dtype=torch.int64, device="cuda")
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        ada.append(geom, graphed, gs, cb8, cb4, kb, vb, sb, th_d, pb)
    torch.cuda.synchronize()
    for step in range(24):
        k, v, sc = _new_tokens(cfg, step, 2)
        pos = torch.tensor([lens[0] + step, lens[1] + step], dtype=torch.int64, device="cuda")
        kb.copy_(k.cuda())
        vb.copy_(v.cuda())
        sb.copy_(sc.cuda())
        pb.copy_(pos)
        g.replay()
        ada.append(geom, eager, es, cb8, cb4, to_dev(k), to_dev(v), to_dev(sc), th_d, pos)
        torch.cuda.synchronize()
        assert torch.equal(graphed.num_pages, eager.num_pages) and torch.equal(graphed.page_meta, eager.page_meta)
        assert torch.equal(graphed.tier_tokens, eager.tier_tokens)
    assert es.pull() == 0 and gs.pull() == 0
    assert int(graphed.cursor[0]) == int(eager.cursor[0])
    # same pages in every row (offsets may differ: rows race for the cursor)
    pt_g = graphed.page_table.cpu().numpy().view(np.uint32)
    pt_e = eager.page_table.cpu().numpy().view(np.uint32)
    ag, ae = graphed.arena.cpu().numpy(), eager.arena.cpu().numpy()
    pm = eager.page_meta.cpu().numpy()
    for row in range(4):
        for p in range(int(eager.num_pages[row])):
            n = ada.page_bytes(128, int(pm[row, p]) & 3)
            assert np.array_equal(ag[int(pt_g[row, p]) * 128:][:n], ae[int(pt_e[row, p]) * 128:][:n])


def _bytes_per_seq(hc, S, H):
    return [sum(oracle.page_bytes(hc.D, int(hc.page_meta[r, p]) & 3)
                for r in range(s * H, s * H + H) for p in range(hc.num_pages[r])) for s in range(S)]


@pytest.mark.parametrize("D,demote_to", [(128, 2), (64, 1)])
def test_decode_loop_with_retiering_under_a_fixed_budget(D, demote_to):
    """Decode steps append one token per sequence; every 16 steps the pages
    are re-tiered to the budget (plan on the host, demotion and eviction on
    the device).  GPU and oracle run the same loop; rows, counters, open
    pages and decode outputs match throughout."""
    cfg = small_workload(D=D, Hq=8, Hkv=2, S=2, T=200, seed=240 + D)
    lens = [200, 120]
    case, hc, _, _ = _base(cfg, lens, 100, 8)
    S, H = 2, 2
    neg = np.full(S, -np.inf, np.float32)   # appends keep fp16; re-tiering does the rest
    budgets = np.array(_bytes_per_seq(hc, S, H), np.int64) * 9 // 10
    geom = geom_of(cfg)
    dc = _upload(hc, geom)
    state = ada.AppendState(geom, dc)
    open_page = np.zeros((S * H, 3), np.int32)
    cb8, cb4 = to_dev(case["cb8"]), to_dev(case["cb4"])
    for step in range(64):
        k, v, sc = _new_tokens(cfg, step, S)
        pos = np.array(lens, np.int64) + step
        ada.append(geom, dc, state, cb8, cb4, to_dev(k), to_dev(v), to_dev(sc), to_dev(neg), to_dev(pos))
        _, st = oracle.append(hc, k, v, sc.numpy(), case["cb8"], case["cb4"], neg, pos, open_page)
        assert st == 0
        if step % 16 == 15:
            assert state.pull() == 0
            rows, pages, tgt = ada.retier_plan(geom, budgets, dc.num_pages_host,
                                               dc.page_meta.cpu().numpy(), demote_to=demote_to)
            o = oracle.retier_plan(hc, budgets, demote_to=demote_to)
            assert all(np.array_equal(x, y) for x, y in zip((rows, pages, tgt), o))
            flush(f"[retier] D={D} step {step}: {len(rows)} pages ({np.bincount(tgt, minlength=4)[1:]})")
            ada.retier(geom, dc, state, cb8, cb4, to_dev(rows), to_dev(pages), to_dev(tgt))
            assert oracle.retier(hc, case["cb8"], case["cb4"], rows, pages, tgt, open_page) == 0
            assert state.pull() == 0
            _compare(dc, hc, f"retier step {step}")
            assert np.array_equal(state.buf[256:256 + 12 * 4].cpu().numpy().view(np.int32).reshape(4, 3),
                                  open_page)
    assert int(dc.cursor[0]) == int(hc.cursor[0])
    now = _bytes_per_seq(hc, S, H)
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, nthreads=8)
    out, lse, _ = decode_outputs(geom, dc, to_dev(case["q"]), with_logits=False)
    ada.decode(geom, dc, cb8, cb4, to_dev(case["q"]), cfg.sigma, out, lse)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().double().numpy() - ref["out"]).max() <= OUT_TOL
    flush(f"[retier] final bytes {now} vs budgets {list(budgets)}")
