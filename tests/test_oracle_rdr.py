"""Pins for the oracle's RDR pieces (CPU only): the angular error of the
stored codes, the budget solver and pack with given tiers.

code_error: closed forms on one-hot keys and zero keys, scale invariance,
and agreement with the encode's own candidate distances (pinned in
test_oracle_encode).  rdr_solve: a hand-worked golden, brute force over all
assignments of tiny problems (the result is optimal among every assignment
of no more bytes -- the Lagrangian property), the budget extremes, the
protection constraint, the reduction to utility ranking when every state has
the same radius and errors, monotonicity in the budget and the strict cap.
pack_tiers: reproduces pack() bit for bit when given the tiers pack() chose.
"""
import itertools
import json
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import make_case, oracle_cache, small_workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f16(x):
    return np.asarray(x, dtype=np.float16).view(np.uint16)


# ---- code_error -------------------------------------------------------------

def _codebooks(H, G, rng):
    cb8 = rng.standard_normal((H, G, 256, 8)).astype(np.float32) * 0.3
    cb4 = rng.standard_normal((H, G, 16, 8)).astype(np.float32) * 0.3
    return cb8, cb4


def test_code_error_closed_form_one_hot_keys():
    D, G = 64, 8
    rng = np.random.default_rng(0)
    cb8, cb4 = _codebooks(1, G, rng)
    # key 3 e_5: u = e_5 (group 0, coordinate 5), every other group u_g = 0
    key = np.zeros((1, 1, D), np.float16)
    key[0, 0, 5] = 3.0
    cb8[0, 0, 7] = 0.0
    cb8[0, 0, 7, 5] = 0.75          # distance 0.25^2
    cb8[0, 1:, 0] = 0.0             # zero codewords elsewhere
    cb4[0, 0, 2] = 0.0
    cb4[0, 0, 2, 5] = 0.5
    cb4[0, 0, 2, 0] = 0.5           # distance 0.25 + 0.25
    cb4[0, 1:, 3] = 0.0
    cb4[0, 1:, 3, 1] = 0.125        # distance 1/64 in each of 7 groups
    c8 = np.zeros((1, 1, G), np.uint8)
    c8[0, 0, 0] = 7
    c4 = np.zeros((1, 1, G // 2), np.uint8)
    c4[0, 0, :] = 0x33
    c4[0, 0, 0] = 0x32              # group 0 -> code 2, group 1 -> code 3
    e8, e4 = oracle.code_error(key, cb8, cb4, c8, c4)
    assert e8[0, 0] == np.float32(0.0625)
    assert e4[0, 0] == np.float32(0.5 + 7 / 64)


def test_code_error_zero_key_is_codeword_energy():
    D, G = 128, 16
    rng = np.random.default_rng(1)
    cb8, cb4 = _codebooks(2, G, rng)
    key = np.zeros((1, 2, D), np.float16)
    c8 = rng.integers(0, 256, (1, 2, G)).astype(np.uint8)
    c4 = rng.integers(0, 256, (1, 2, G // 2)).astype(np.uint8)
    e8, e4 = oracle.code_error(key, cb8, cb4, c8, c4)
    for h in range(2):
        w8 = sum(float(np.sum(cb8[h, g, c8[0, h, g]].astype(np.float64) ** 2)) for g in range(G))
        c4g = [(c4[0, h, g // 2] >> (4 * (g % 2))) & 15 for g in range(G)]
        w4 = sum(float(np.sum(cb4[h, g, c4g[g]].astype(np.float64) ** 2)) for g in range(G))
        assert abs(e8[0, h] - w8) <= 1e-6 * w8 and abs(e4[0, h] - w4) <= 1e-6 * w4


def test_code_error_matches_encode_distances_and_is_scale_invariant():
    cfg = small_workload(D=128, Hq=4, Hkv=2, T=40, seed=5)
    case = make_case(cfg)
    k = case["keys"]
    r, c8, c4, d8, d4 = oracle.encode(k, case["cb8"], case["cb4"], with_dist=True)
    e8, e4 = oracle.code_error(k, case["cb8"], case["cb4"], c8, c4)
    N, H, G = c8.shape
    for n in range(N):
        for h in range(H):
            s8 = s4 = 0.0
            for g in range(G):
                s8 += d8[n, h, g, c8[n, h, g]]
                s4 += d4[n, h, g, (c4[n, h, g // 2] >> (4 * (g % 2))) & 15]
            assert e8[n, h] == np.float32(s8) and e4[n, h] == np.float32(s4)
    assert (e8 <= e4 + 1.0).all() and (e8 >= 0).all()
    k2 = (k.float() * 2).to(torch.float16)  # exact: a power of two, far from overflow
    assert torch.equal(k2.float(), k.float() * 2)
    f8, f4 = oracle.code_error(k2, case["cb8"], case["cb4"], c8, c4)
    assert np.array_equal(f8, e8) and np.array_equal(f4, e4)


# ---- rdr_solve --------------------------------------------------------------

def _rates(D):
    return [oracle.page_bytes(D, t) // 16 for t in range(3)] + [0]


def _distortions(score, radius_bits, e8, e4):
    """D_b per state, in binary32 as the solver defines them."""
    wr = np.float32(score) * np.float32(np.uint16(radius_bits).view(np.float16))
    return [np.float32(0), wr * np.sqrt(np.float32(e8)), wr * np.sqrt(np.float32(e4)), wr]


def test_rdr_solve_golden_hand_cases():
    with open(os.path.join(GOLDEN, "rdr_solve_hand.json")) as f:
        g = json.load(f)
    D = g["D"]
    st = g["states"]
    n = len(st)
    cu = np.array([0, n], np.int32)
    r = _f16([[x["radius"]] for x in st])
    e8 = np.array([[x["err8"]] for x in st], np.float32)
    e4 = np.array([[x["err4"]] for x in st], np.float32)
    sc = np.array([[x["score"]] for x in st], np.float32)
    reserve = 15 * sum(_rates(D)[:3])
    for case in g["cases"]:
        pr = None if "protect" not in case else np.array(case["protect"], np.uint8).reshape(n, 1)
        t = oracle.rdr_solve(D, cu, [case["cap"] + reserve], r, e8, e4, sc, protect=pr)
        assert t.ravel().tolist() == case["tiers"], case["note"]


def _brute(D, R, Dist, prot, cap):
    """Every assignment: (rate, distortion) pairs (tiny problems only)."""
    n = len(Dist)
    opts = [[0] if prot[i] else [0, 1, 2, 3] for i in range(n)]
    out = []
    for a in itertools.product(*opts):
        rate = sum(R[b] for b in a)
        dist = sum(float(Dist[i][b]) for i, b in enumerate(a))
        out.append((rate, dist, a))
    return out


@pytest.mark.parametrize("seed", range(12))
def test_rdr_solve_is_optimal_for_its_own_rate_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    D = 64 if seed % 2 else 128
    H, T = (1, 5) if seed % 3 else (2, 3)
    n = H * T
    R = _rates(D)
    r = _f16(rng.uniform(0.1, 20, (T, H)))
    e8 = rng.uniform(0.01, 0.6, (T, H)).astype(np.float32)
    e4 = (e8 + rng.uniform(-0.05, 0.6, (T, H))).clip(0.0, 2.0).astype(np.float32)
    sc = rng.integers(1, 50, (T, H)).astype(np.float32)
    prot = (rng.random((T, H)) < 0.15).astype(np.uint8)
    flat = [(t, h) for t in range(T) for h in range(H)]
    Dist = [_distortions(sc[t, h], r[t, h], e8[t, h], e4[t, h]) for t, h in flat]
    pflat = [int(prot[t, h]) for t, h in flat]
    reserve = H * 15 * sum(R[:3])
    allv = None
    for cap in rng.integers(-50, n * R[0] + 50, 6):
        t = oracle.rdr_solve(D, [0, T], [int(cap) + reserve], r, e8, e4, sc, protect=prot)
        a = [int(t[i, j]) for i, j in flat]
        assert all(a[i] == 0 for i in range(n) if pflat[i])
        rate = sum(R[b] for b in a)
        dist = sum(float(Dist[i][b]) for i, b in enumerate(a))
        allv = allv or _brute(D, R, Dist, pflat, cap)
        min_rate = min(x[0] for x in allv)
        if min_rate <= cap:
            assert rate <= cap
        else:
            assert a == [0 if p else 3 for p in pflat]  # infeasible: drop all unprotected
        best = min(x[1] for x in allv if x[0] <= rate)
        assert dist <= best * (1 + 1e-5) + 1e-6, (dist, best)


def test_rdr_solve_budget_extremes_and_protection():
    rng = np.random.default_rng(7)
    T, H, D = 300, 4, 128
    R = _rates(D)
    cu = np.array([0, 100, 300], np.int32)
    r = _f16(rng.uniform(0.5, 30, (T, H)))
    e8 = rng.uniform(0.02, 0.5, (T, H)).astype(np.float32)
    e4 = rng.uniform(0.2, 0.9, (T, H)).astype(np.float32)
    sc = rng.integers(1, 1000, (T, H)).astype(np.float32)
    reserve = H * 15 * sum(R[:3])
    full = [100 * H * R[0] + reserve, 200 * H * R[0] + reserve]
    assert (oracle.rdr_solve(D, cu, full, r, e8, e4, sc) == 0).all()
    assert (oracle.rdr_solve(D, cu, [0, 0], r, e8, e4, sc) == 3).all()
    prot = (rng.random((T, H)) < 0.1).astype(np.uint8)
    t = oracle.rdr_solve(D, cu, [0, 0], r, e8, e4, sc, protect=prot)
    assert np.array_equal(t, np.where(prot == 1, 0, 3).astype(np.uint8))
    t = oracle.rdr_solve(D, cu, [f // 2 for f in full], r, e8, e4, sc, protect=prot)
    assert (t[prot == 1] == 0).all()


def test_rdr_solve_reduces_to_utility_ranking_with_equal_errors():
    """Same radius and errors everywhere: the chains differ only by the
    score factor, so the solver keeps the higher-utility states at the
    higher tiers, i.e. the ranking rule of pack() with the solver's counts."""
    rng = np.random.default_rng(8)
    T, D = 400, 64
    R = _rates(D)
    cu = np.array([0, T], np.int32)
    r = _f16(np.full((T, 1), 2.0))
    e8 = np.full((T, 1), 0.09, np.float32)
    e4 = np.full((T, 1), 0.36, np.float32)
    sc = rng.permutation(T).astype(np.float32).reshape(T, 1) + 1.0
    reserve = 15 * sum(R[:3])
    for frac in (0.2, 0.45, 0.7):
        t = oracle.rdr_solve(D, cu, [int(frac * T * R[0]) + reserve], r, e8, e4, sc)[:, 0]
        order = np.argsort(-sc[:, 0], kind="stable")
        assert (np.diff(t[order].astype(int)) >= 0).all()  # tiers non-decreasing down the ranking
        cnt = np.bincount(t, minlength=4)
        bp = None  # the rank rule with these counts gives the same assignment
        ranked = np.repeat(np.arange(4), cnt)
        assert np.array_equal(t[order], ranked)


def test_rdr_solve_monotone_in_budget_and_strict_cap():
    rng = np.random.default_rng(9)
    T, H, D = 500, 2, 128
    R = np.array(_rates(D))
    cu = np.array([0, T], np.int32)
    r = _f16(rng.uniform(0.5, 30, (T, H)))
    e8 = rng.uniform(0.02, 0.5, (T, H)).astype(np.float32)
    e4 = rng.uniform(0.2, 0.9, (T, H)).astype(np.float32)
    sc = rng.integers(1, 1000, (T, H)).astype(np.float32)
    Dist = np.array([[_distortions(sc[t, h], r[t, h], e8[t, h], e4[t, h]) for h in range(H)]
                     for t in range(T)], np.float64)
    prev = None
    for frac in np.linspace(0.05, 1.05, 21):
        budget = int(frac * T * H * R[0])
        t = oracle.rdr_solve(D, cu, [budget], r, e8, e4, sc)
        rate = int(R[t].sum())
        dist = float(np.take_along_axis(Dist, t[..., None].astype(np.int64), 2).sum())
        pages = sum(oracle.page_bytes(D, k) * -(-int((t[:, h] == k).sum()) // 16)
                    for h in range(H) for k in range(3))
        assert pages <= budget or (t == 3).all()
        if prev is not None:
            assert rate >= prev[0] and dist <= prev[1] * (1 + 1e-6)
        prev = (rate, dist)


# ---- pack_tiers ---------------------------------------------------------------

def test_pack_tiers_reproduces_pack_from_its_own_tiers():
    cfg = small_workload(D=128, Hq=4, Hkv=2, S=3, T=300, seed=12)
    case = make_case(cfg, lens=[300, 47, 0], mixes=[(1500, 6000, 8500), (1500, 5000, 10000), (0, 0, 0)])
    prot = (np.random.default_rng(3).random((case["N"], 2)) < 0.03).astype(np.uint8)
    hc, (r, c8, c4) = oracle_cache(case, protect=prot)
    # the tier pack() gave every (token, head), read back from the pages
    tiers = np.full((case["N"], 2), 3, np.uint8)
    for row in range(hc.S * hc.Hkv):
        s, h = divmod(row, hc.Hkv)
        for p in range(hc.num_pages[row]):
            tier = hc.page_meta[row, p] & 3
            for tok in hc.slot_token[row, p]:
                if tok >= 0:
                    tiers[case["cu"][s] + tok, h] = tier
    hc2 = oracle.HostCache(hc.D, hc.Hkv, hc.S, hc.maxp, len(hc.arena))
    assert oracle.pack_tiers(hc2, case["cu"], tiers, case["keys"], case["values"], r, c8, c4) == 0
    for name in ("arena", "page_table", "page_meta", "num_pages", "tier_tokens", "slot_token"):
        assert np.array_equal(getattr(hc, name), getattr(hc2, name)), name
    assert np.array_equal(oracle.row_tier_counts(case["cu"], tiers), hc.tier_tokens)


def test_pack_tiers_places_every_kept_state_once():
    cfg = small_workload(D=64, Hq=2, Hkv=2, S=2, T=90, seed=13)
    case = make_case(cfg, lens=[90, 33])
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    tiers = np.random.default_rng(4).integers(0, 4, (case["N"], 2)).astype(np.uint8)
    hc = oracle.HostCache(64, 2, 2, 16, 1 << 20)
    assert oracle.pack_tiers(hc, case["cu"], tiers, case["keys"], case["values"], r, c8, c4) == 0
    seen = np.zeros((case["N"], 2), np.int32)
    for row in range(4):
        s, h = divmod(row, 2)
        for p in range(hc.num_pages[row]):
            tier = hc.page_meta[row, p] & 3
            for tok in hc.slot_token[row, p]:
                if tok >= 0:
                    assert tiers[case["cu"][s] + tok, h] == tier
                    seen[case["cu"][s] + tok, h] += 1
    assert np.array_equal(seen, (tiers < 3).astype(np.int32))
    # a value other than the kept tiers 0-2 means not resident (the residency
    # bit of the technical summary, section 2.2), exactly like 3
    odd = np.where(tiers == 3, 200, tiers).astype(np.uint8)
    hc3 = oracle.HostCache(64, 2, 2, 16, 1 << 20)
    assert oracle.pack_tiers(hc3, case["cu"], odd, case["keys"], case["values"], r, c8, c4) == 0
    assert np.array_equal(hc3.arena, hc.arena) and np.array_equal(hc3.slot_token, hc.slot_token)
