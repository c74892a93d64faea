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
