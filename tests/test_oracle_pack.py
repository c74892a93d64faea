"""Pins for the oracle's RDR pack (tiering + tier-homogeneous pages), CPU only.

Pinned by the invariants the pages and the reading fix: every retained
(token, head) appears once and dropped ones never; tier sizes follow the
counts; every page holds one tier; ranking by utility (protected first);
unpacked fields equal the inputs; padding is zero; placement follows the
given order."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from helpers import f16_bits_to_f64, make_case, small_workload
from pagefmt import read_page

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_tier_counts_golden():
    with open(os.path.join(GOLDEN, "tier_counts.json")) as f:
        g = json.load(f)
    for c in g["cases"]:
        assert list(oracle.tier_counts(c["T"], c["bp"])) == c["n_cum"], c["note"]


def _u16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def _check_cache(cache, case, enc, calls, protect=None):
    """calls: list of (cu, bp, token offset of the call, pos_base)."""
    D, H = cache.D, cache.Hkv
    G = D // 8
    r, c8, c4 = enc
    keys, vals = _u16(case["keys"]), _u16(case["values"])
    scores = case["scores"].numpy()
    S = cache.S
    seen = {}
    for row in range(S * H):
        s, h = divmod(row, H)
        tiers = (cache.page_meta[row, : cache.num_pages[row]] & 3).astype(int)
        for p in range(cache.num_pages[row]):
            meta = int(cache.page_meta[row, p])
            tier, nv = meta & 3, ((meta >> 2) & 15) + 1
            pg = read_page(cache.page(row, p), D, tier)
            assert not pg["pad"].any()
            for t in range(16):
                tok = int(cache.slot_token[row, p, t])
                if t >= nv:
                    assert tok == -1
                    for k, v in pg.items():
                        if k != "pad" and v.ndim >= 1 and v.shape[0] == 16:
                            assert not np.asarray(v[t]).any()
                    continue
                assert (tok, h) not in seen
                seen[(tok, h)] = tier
                e = tok  # flat index of the token in this case's arrays
                if tier == 0:
                    assert np.array_equal(pg["K"][t], keys[e, h])
                    assert np.array_equal(pg["V"][t], vals[e, h])
                elif tier == 1:
                    assert np.array_equal(pg["V"][t], vals[e, h])
                    assert np.array_equal(pg["codes"][t], c8[e, h])
                    assert pg["radius"][t] == r[e, h]
                else:
                    assert np.array_equal(pg["codes4"][t], c4[e, h])
                    assert pg["radius"][t] == r[e, h]
                    q, sc = oracle.quant_v(vals[e, h])
                    assert np.array_equal(pg["Vq"][t], q) and pg["vscale"][t] == sc
        # pages of one call: fp16, then 8-bit, then 4-bit (non-decreasing tier)
        # within each call's block of pages
        del tiers
    # per call: tier sizes, score order, protected -> fp16, dropped absent
    for cu, bp, off, pos_base in calls:
        for s in range(S):
            T = int(cu[s + 1] - cu[s])
            n = oracle.tier_counts(T, bp[s])
            for h in range(H):
                toks = [pos_base[s] + i for i in range(T)]
                flat = [off + cu[s] + i for i in range(T)]
                got = [seen.get((f, h), 3) for f in flat]
                sizes = [got.count(k) for k in range(4)]
                assert sizes == [n[0], n[1] - n[0], n[2] - n[1], T - n[2]]
                # ranking: key (protect, score, -idx) strictly decreases across tiers
                keyf = [((protect[f, h] if protect is not None else 0), scores[f, h], -i)
                        for i, f in enumerate(flat)]
                for a in range(T):
                    for b in range(T):
                        if got[a] < got[b]:
                            assert keyf[a] > keyf[b]
                if protect is not None:
                    for i, f in enumerate(flat):
                        if protect[f, h]:
                            assert got[i] == 0
                del toks
    return seen


def _perm(n, seed):
    return np.random.default_rng(seed).permutation(n).astype(np.uint32)


@pytest.mark.parametrize("D", [64, 128])
def test_pack_invariants_two_calls_protect_and_permuted_pool(D):
    cfg = small_workload(D=D, Hq=4, Hkv=2, S=3, T=100, seed=10 + D)
    lens1 = np.array([100, 37, 0])
    lens2 = np.array([20, 0, 45])
    case = make_case(cfg, lens=np.concatenate([lens1, lens2]),
                     mixes=[(2500, 7500, 9000)] * 6)
    N1 = int(lens1.sum())
    enc = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    r, c8, c4 = enc
    H = cfg.num_kv_heads
    rng = np.random.default_rng(D)
    protect = (rng.random((case["N"], H)) < 0.05).astype(np.uint8)
    # scores with many ties so the index tie-break matters
    scores = torch.from_numpy(rng.integers(1, 4, (case["N"], H)).astype(np.float32))
    case["scores"] = scores
    cache = oracle.HostCache(D, H, 3, 20, 1 << 20)
    bp1 = np.array([(2500, 7500, 9000), (0, 5000, 10000), (3000, 3000, 3000)], np.int32)
    cu1 = np.array([0, 100, 137, 137], np.int32)
    # protected tokens must fit in each sequence's fp16 count
    for s in range(3):
        n0 = oracle.tier_counts(cu1[s + 1] - cu1[s], bp1[s])[0]
        for h in range(H):
            sl = protect[cu1[s]:cu1[s + 1], h]
            idx = np.nonzero(sl)[0]
            sl[idx[n0:]] = 0
    n_pages1 = oracle.num_pages_of_call(D, H, cu1, bp1)
    rc = oracle.pack(cache, cu1, bp1, case["keys"][:N1], case["values"][:N1], r[:N1], c8[:N1],
                     c4[:N1], scores[:N1], protect=protect[:N1], place_perm=_perm(n_pages1, 1))
    assert rc == 0
    first_call_pages = cache.num_pages.copy()
    # second call appends to the same rows; its token indices continue each sequence
    bp2 = np.array([(10000, 10000, 10000), (5000, 5000, 5000), (0, 2000, 6000)], np.int32)
    cu2 = np.array([0, 20, 20, 65], np.int32)
    pos2 = np.array([100, 37, 0], np.int64)
    sl = slice(N1, None)
    n_pages2 = oracle.num_pages_of_call(D, H, cu2, bp2)
    # slot_token records pos_base + index; map it back to flat indices below
    protect[N1:] = 0
    rc = oracle.pack(cache, cu2, bp2, case["keys"][sl], case["values"][sl], r[sl], c8[sl], c4[sl],
                     scores[sl], protect=protect[N1:],
                     place_perm=_perm(n_pages2, 2), pos_base=pos2)
    assert rc == 0
    # translate recorded positions to flat indices for checking
    st = cache.slot_token.copy()
    for row in range(3 * H):
        s = row // H
        for p in range(cache.num_pages[row]):
            for t in range(16):
                v = st[row, p, t]
                if v < 0:
                    continue
                if p >= first_call_pages[row]:
                    st[row, p, t] = N1 + cu2[s] + (v - pos2[s])
                else:
                    st[row, p, t] = cu1[s] + v
    cache_view = cache
    saved = cache.slot_token
    cache_view.slot_token = st
    _check_cache(cache_view, case, enc,
                 [(cu1, bp1, 0, [0, 0, 0]), (cu2, bp2, N1, list(pos2))], protect=protect)
    cache.slot_token = saved
    # placement: the call's pages are contiguous in the arena in permuted order
    total = int(cache.cursor[0])
    offs = sorted((int(cache.page_table[r_, p]), r_, p)
                  for r_ in range(3 * H) for p in range(cache.num_pages[r_]))
    cur = 0
    for off, r_, p in offs:
        assert off == cur
        cur += oracle.page_bytes(D, int(cache.page_meta[r_, p]) & 3) // 128
    assert cur == total


def test_pack_single_tier_pages_and_order():
    cfg = small_workload(D=64, Hq=4, Hkv=2, S=2, T=77, seed=5)
    case = make_case(cfg, mixes=[(2000, 6000, 9000), (1000, 1000, 8000)])
    cache, _ = __import__("helpers").oracle_cache(case)
    for row in range(cache.S * cache.Hkv):
        tiers = [int(m) & 3 for m in cache.page_meta[row, : cache.num_pages[row]]]
        assert tiers == sorted(tiers)
        tt = cache.tier_tokens[row]
        s = row // cache.Hkv
        n = oracle.tier_counts(77, case["bp"][s])
        assert list(tt) == [n[0], n[1] - n[0], n[2] - n[1]]


def test_pack_errors_leave_cache_untouched():
    cfg = small_workload(D=64, Hq=4, Hkv=2, S=1, T=64, seed=6)
    case = make_case(cfg)
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    args = (case["cu"], case["bp"], case["keys"], case["values"], r, c8, c4, case["scores"])
    # arena too small
    small = oracle.HostCache(64, 2, 1, 16, 4096)
    assert oracle.pack(small, *args) == 3
    assert small.cursor[0] == 0 and not small.num_pages.any() and not small.arena.any()
    # page-table rows too short
    short = oracle.HostCache(64, 2, 1, 2, 1 << 20)
    assert oracle.pack(short, *args) == 1
    assert short.cursor[0] == 0 and not short.num_pages.any()
    # more protected tokens than the fp16 tier holds (25% of 64 = 16)
    prot = np.zeros((64, 2), np.uint8)
    prot[:17, 0] = 1
    c = oracle.HostCache(64, 2, 1, 16, 1 << 20)
    assert oracle.pack(c, *args, protect=prot) == 1
    assert c.cursor[0] == 0
    # decreasing cumulative basis points
    c = oracle.HostCache(64, 2, 1, 16, 1 << 20)
    bad = np.array([[5000, 4000, 10000]], np.int32)
    assert oracle.pack(c, case["cu"], bad, *args[2:]) == 1
    # placement order that is not a permutation
    n = oracle.num_pages_of_call(64, 2, case["cu"], case["bp"])
    c = oracle.HostCache(64, 2, 1, 16, 1 << 20)
    assert oracle.pack(c, *args, place_perm=np.zeros(n, np.uint32)) == 1


def test_value_dequant_error_bound_in_pages():
    cfg = small_workload(D=128, Hq=4, Hkv=1, S=1, T=48, mix=(0, 0, 10000), seed=7)
    case = make_case(cfg)
    cache, _ = __import__("helpers").oracle_cache(case)
    vals = case["values"].double().numpy()
    for p in range(cache.num_pages[0]):
        pg = read_page(cache.page(0, p), 128, 2)
        for t in range(16):
            tok = cache.slot_token[0, p, t]
            if tok < 0:
                continue
            s = f16_bits_to_f64(pg["vscale"][t:t + 1])[0]
            vhat = pg["Vq"][t].astype(np.float64) * s
            amax = np.abs(vals[tok, 0]).max()
            assert np.abs(vhat - vals[tok, 0]).max() <= 0.5 * s + amax * 2.0 ** -10
