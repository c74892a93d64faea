"""Pins for the oracle's decode-step append (CPU only).

Appending tokens one decode step at a time with the slope threshold of a
solve over the same tokens gives every token the tier the solve gave it;
with an all-fp16 threshold the pages equal pack()'s; with any tiers each
row holds the same pages (as byte strings) as pack_tiers() builds, and
decodes to the same outputs; full page tables and a full arena set the
status bits and store nothing out of place."""
import numpy as np
import pytest
import torch

import oracle
import synth
from helpers import make_case, small_workload


def _steps(case, T):
    """Token t of every sequence as one decode step: [S][Hkv][D] slices."""
    S = len(case["lens"])
    cu = case["cu"]
    for t in range(T):
        idx = [int(cu[s]) + t for s in range(S)]
        yield t, idx


def _row_pages(hc, row):
    out = []
    for p in range(hc.num_pages[row]):
        out.append((int(hc.page_meta[row, p]), hc.page(row, p).tobytes(),
                    tuple(hc.slot_token[row, p]) if hc.slot_token is not None else None))
    return out


def _append_all(case, cfg, threshold, maxp, arena, protect=None):
    S, H = len(case["lens"]), cfg.num_kv_heads
    T = int(case["lens"][0])
    hc = oracle.HostCache(cfg.head_dim, H, S, maxp, arena)
    open_page = np.zeros((S * H, 3), np.int32)
    tiers = np.zeros((case["N"], H), np.uint8)
    status = 0
    for t, idx in _steps(case, T):
        pr = None if protect is None else protect[idx]
        tt, st = oracle.append(hc, case["keys"][idx], case["values"][idx], case["scores"][idx].numpy(),
                               case["cb8"], case["cb4"], threshold, np.full(S, t, np.int64), open_page,
                               protect=pr)
        tiers[idx] = tt
        status |= st
    return hc, tiers, status


@pytest.mark.parametrize("D", [64, 128])
def test_append_tiers_equal_the_solve_over_the_same_tokens(D):
    cfg = small_workload(D=D, Hq=4, Hkv=2, S=3, T=160, seed=30 + D)
    case = make_case(cfg, lens=[160, 160, 160])
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    e8, e4 = oracle.code_error(case["keys"], case["cb8"], case["cb4"], c8, c4)
    prot = (np.random.default_rng(D).random((case["N"], 2)) < 0.05).astype(np.uint8)
    budgets = synth.budget_bytes(cfg, case["lens"]) * np.array([3, 5, 9]) // 10
    tiers, th = oracle.rdr_solve(D, case["cu"], budgets, r, e8, e4, case["scores"].numpy(), protect=prot,
                                 with_threshold=True)
    hc, got, status = _append_all(case, cfg, th, 40, 1 << 22, protect=prot)
    assert status == 0
    assert np.array_equal(got, tiers)
    # and the pages are those pack_tiers builds from the same tiers
    ref = oracle.HostCache(D, 2, 3, 40, 1 << 22)
    assert oracle.pack_tiers(ref, case["cu"], tiers, case["keys"], case["values"], r, c8, c4,
                             pos_base=np.zeros(3, np.int64)) == 0
    for row in range(6):
        assert sorted(_row_pages(hc, row)) == sorted(_row_pages(ref, row))
    assert np.array_equal(hc.tier_tokens, ref.tier_tokens) and np.array_equal(hc.num_pages, ref.num_pages)
    a = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    b = oracle.decode(ref, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    assert np.abs(a["out"] - b["out"]).max() < 1e-12 and np.allclose(a["lse"], b["lse"], rtol=1e-13)


def test_append_at_fp16_equals_pack_of_all_tokens():
    cfg = small_workload(D=128, Hq=2, Hkv=2, S=2, T=50, seed=33)
    case = make_case(cfg, lens=[50, 50])
    hc, tiers, status = _append_all(case, cfg, np.full(2, -np.inf, np.float32), 8, 1 << 21)
    assert status == 0 and (tiers == 0).all()
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    ref = oracle.HostCache(128, 2, 2, 8, 1 << 21)
    assert oracle.pack(ref, case["cu"], [[10000] * 3] * 2, case["keys"], case["values"], r, c8, c4,
                       case["scores"]) == 0
    for row in range(4):
        assert _row_pages(hc, row) == _row_pages(ref, row)  # same order too: 16, 16, 16, 2 slots
    # +inf drops every unprotected state
    hc2, t2, st2 = _append_all(case, cfg, np.full(2, np.inf, np.float32), 8, 1 << 21)
    assert st2 == 0 and (t2 == 3).all() and not hc2.num_pages.any() and hc2.cursor[0] == 0


def test_append_capacity_status_bits():
    cfg = small_workload(D=64, Hq=2, Hkv=2, S=2, T=40, seed=34)
    case = make_case(cfg, lens=[40, 40])
    # two pages per row only: the third page of every row is refused
    hc, _, st = _append_all(case, cfg, np.full(2, -np.inf, np.float32), 2, 1 << 20)
    assert st == 1 and (hc.num_pages == 2).all() and (hc.tier_tokens[:, 0] == 32).all()
    # arena for three fp16 pages (32 units each at D = 64)
    hc, _, st = _append_all(case, cfg, np.full(2, -np.inf, np.float32), 8, 3 * 4096)
    assert st == 2 and int(hc.num_pages.sum()) == 3 and hc.cursor[0] == 96


def _packed(case, cfg, tiers, maxp=40):
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    hc = oracle.HostCache(cfg.head_dim, cfg.num_kv_heads, len(case["lens"]), maxp, 1 << 22)
    assert oracle.pack_tiers(hc, case["cu"], tiers, case["keys"], case["values"], r, c8, c4) == 0
    return hc


@pytest.mark.parametrize("tier", [1, 2])
def test_retier_demotion_equals_packing_at_that_tier(tier):
    """Demoting fp16 pages re-encodes their keys from the page itself: the
    result is the page pack_tiers builds for the same tokens at that tier."""
    cfg = small_workload(D=128, Hq=4, Hkv=2, S=2, T=70, seed=40 + tier)
    case = make_case(cfg, lens=[70, 33])
    fp16 = _packed(case, cfg, np.zeros((case["N"], 2), np.uint8))
    coded = _packed(case, cfg, np.full((case["N"], 2), tier, np.uint8))
    rows, pages = np.nonzero(np.arange(fp16.maxp)[None, :] < fp16.num_pages[:, None])
    open_page = np.zeros((4, 3), np.int32)
    st = oracle.retier(fp16, case["cb8"], case["cb4"], rows, pages, np.full(len(rows), tier), open_page)
    assert st == 0
    for row in range(4):
        assert _row_pages(fp16, row) == _row_pages(coded, row)
    assert np.array_equal(fp16.tier_tokens, coded.tier_tokens)
    # demoting a page that is not fp16 is refused and changes nothing
    before = (fp16.page_table.copy(), fp16.page_meta.copy(), fp16.cursor.copy())
    assert oracle.retier(fp16, case["cb8"], case["cb4"], [0], [0], [2], open_page) == 4
    assert np.array_equal(before[0], fp16.page_table) and before[2][0] == fp16.cursor[0]


def test_retier_eviction_keeps_the_other_pages_and_remaps_open_pages():
    cfg = small_workload(D=64, Hq=2, Hkv=2, S=1, T=120, seed=45)
    case = make_case(cfg, lens=[120])
    rng = np.random.default_rng(45)
    tiers = rng.integers(0, 3, (120, 2)).astype(np.uint8)
    hc = _packed(case, cfg, tiers)
    before = [_row_pages(hc, row) for row in range(2)]
    n0 = hc.num_pages.copy()
    open_page = np.array([[n0[0], 0, 0], [0, 0, n0[1]]], np.int32)  # each row's last page is open
    ev0 = [0, int(n0[0]) - 1, 2]
    ev1 = [int(n0[1]) - 2]
    st = oracle.retier(hc, case["cb8"], case["cb4"], [0, 1, 0, 0], [ev0[0], ev1[0], ev0[1], ev0[2]],
                       [3, 3, 3, 3], open_page)
    assert st == 0
    for row, ev in ((0, ev0), (1, ev1)):
        kept = [pg for i, pg in enumerate(before[row]) if i not in ev]
        assert sorted(_row_pages(hc, row)) == sorted(kept)
        assert hc.num_pages[row] == n0[row] - len(ev)
        counts = np.zeros(3, np.int64)
        for meta, _, _ in kept:
            counts[meta & 3] += ((meta >> 2) & 15) + 1
        assert np.array_equal(hc.tier_tokens[row], counts)
    assert open_page[0, 0] == 0                     # row 0's open page was evicted
    last1 = before[1][-1]
    assert _row_pages(hc, 1)[open_page[1, 2] - 1] == last1   # row 1's open page moved, still open


def test_retier_plan_brings_sequences_under_budget_oldest_first():
    cfg = small_workload(D=128, Hq=4, Hkv=2, S=2, T=400, seed=46)
    case = make_case(cfg, lens=[400, 250])
    hc = _packed(case, cfg, np.zeros((case["N"], 2), np.uint8), maxp=32)
    used = [sum(oracle.page_bytes(128, int(hc.page_meta[r, p]) & 3) for r in rows for p in range(hc.num_pages[r]))
            for rows in ((0, 1), (2, 3))]
    budgets = [int(used[0] * 0.7), int(used[1] * 0.2)]
    rows, pages, tgt = oracle.retier_plan(hc, budgets, demote_to=2)
    # sequence 0: only demotions of its oldest full fp16 pages, oldest first
    s0 = rows < 2
    assert (tgt[s0] == 2).all() and list(zip(pages[s0], rows[s0])) == sorted(zip(pages[s0], rows[s0]))
    open_page = np.zeros((4, 3), np.int32)
    assert oracle.retier(hc, case["cb8"], case["cb4"], rows, pages, tgt, open_page) == 0
    now = [sum(oracle.page_bytes(128, int(hc.page_meta[r, p]) & 3) for r in rr for p in range(hc.num_pages[r]))
           for rr in ((0, 1), (2, 3))]
    assert now[0] <= budgets[0]
    # sequence 1 needs evictions too: a second plan (now seeing coded pages) gets it there
    rows2, pages2, tgt2 = oracle.retier_plan(hc, budgets, demote_to=2)
    assert (rows2 >= 2).all() and (tgt2 == 3).any()
    assert oracle.retier(hc, case["cb8"], case["cb4"], rows2, pages2, tgt2, open_page) == 0
    now = sum(oracle.page_bytes(128, int(hc.page_meta[r, p]) & 3) for r in (2, 3) for p in range(hc.num_pages[r]))
    assert now <= budgets[1]
    assert len(oracle.retier_plan(hc, budgets)[0]) == 0


def test_retier_entries_that_cannot_apply_set_bit4_and_change_nothing():
    """A dense comparison page (tier 3) has no tier count, so it is not
    evicted; rows outside the cache and unknown targets are skipped too.
    Each sets status bit 4 and leaves every table, count and byte as it was."""
    cfg = small_workload(D=64, Hq=2, Hkv=2, S=1, T=50, seed=47)
    case = make_case(cfg, lens=[50])
    hc = oracle.HostCache(64, 2, 1, 8, 1 << 20)
    assert oracle.dense_pack(hc, case["cu"], case["keys"], case["values"]) == 0
    tt0 = np.array([[50, 0, 0], [50, 0, 0]], np.int32)
    hc.tier_tokens[:] = tt0  # (a dense cache keeps no counts; any values must stay)
    snap = (hc.page_table.copy(), hc.page_meta.copy(), hc.num_pages.copy(), hc.arena.copy(),
            hc.tier_tokens.copy(), hc.cursor.copy())
    open_page = np.zeros((2, 3), np.int32)
    for rows, pages, tgt in (([0], [1], [3]),        # evict a tier-3 page
                             ([1], [0], [1]),        # demote a tier-3 page
                             ([2], [0], [3]),        # row past the cache
                             ([-1], [0], [2]),       # negative row
                             ([0], [0], [0]),        # unknown target
                             ([0], [0], [4])):
        assert oracle.retier(hc, case["cb8"], case["cb4"], rows, pages, tgt, open_page) == 4
        for a, b in zip(snap, (hc.page_table, hc.page_meta, hc.num_pages, hc.arena, hc.tier_tokens,
                               hc.cursor)):
            assert np.array_equal(a, b)
    # a valid entry beside a bad one still applies
    cfg2 = small_workload(D=64, Hq=2, Hkv=2, S=1, T=64, seed=48)
    case2 = make_case(cfg2, lens=[64])
    coded = _packed(case2, cfg2, np.full((64, 2), 1, np.uint8))
    n0 = coded.num_pages.copy()
    st = oracle.retier(coded, case2["cb8"], case2["cb4"], [5, 1], [0, 0], [3, 3], np.zeros((2, 3), np.int32))
    assert st == 4 and coded.num_pages[1] == n0[1] - 1 and coded.num_pages[0] == n0[0]
