"""GPU parity of the RDR pieces through the C ABI against the CPU oracle.

Bars: code errors bit-exact (both sides sum the same doubles in the same
order and round once); solver tiers bit-exact given the same inputs (the
decisions are binary32 arithmetic in a fixed order on both sides); tier
counts exact; pages, tables and metadata of rdr_pack_tiers bit-exact; the
decode of a solver-built cache within the decode bars (outputs max-abs
<= 1e-2, lse within 1e-3 * max(|lse|, 1))."""
import json
import os

import numpy as np
import pytest
import torch

import compressed_kv_attention_amd as ada
import oracle
import synth
from gpu_util import decode_outputs, flush, geom_of, gpu_encode, to_dev, u16
from helpers import make_case, small_workload

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
OUT_TOL = 1e-2


def _codes(case):
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"], nthreads=8)
    return r, c8, c4


@pytest.mark.parametrize("D", [64, 128])
def test_code_error_bit_exact(D):
    cfg = small_workload(D=D, Hq=4, Hkv=2, S=2, T=700, seed=80 + D)
    case = make_case(cfg, lens=[700, 333])
    r, c8, c4 = _codes(case)
    rng = np.random.default_rng(D)
    rc8 = rng.integers(0, 256, c8.shape).astype(np.uint8)   # any codes, not only the nearest
    rc4 = rng.integers(0, 256, c4.shape).astype(np.uint8)
    geom = geom_of(cfg)
    k = to_dev(case["keys"])
    cb8, cb4 = to_dev(case["cb8"]), to_dev(case["cb4"])
    for codes8, codes4, label in ((c8, c4, "nearest"), (rc8, rc4, "random")):
        flush(f"[code_error] D={D} {label}")
        e8 = torch.full(c8.shape[:2], float("nan"), device="cuda")
        e4 = torch.full(c8.shape[:2], float("nan"), device="cuda")
        ada.code_error(geom, k, cb8, cb4, to_dev(codes8), to_dev(codes4), e8, e4)
        torch.cuda.synchronize()
        r8, r4 = oracle.code_error(case["keys"], case["cb8"], case["cb4"], codes8, codes4)
        assert np.array_equal(e8.cpu().numpy(), r8) and np.array_equal(e4.cpu().numpy(), r4)



def _extreme_keys(T, H, D, seed):
    """fp16 key bits [T][H][D] over the cases that stress u = k / |k|: zero
    keys (u = 0), one nonzero coordinate (u = +-1), four equal powers of two
    (|k| a power of two), exponents over the whole binary16 range,
    subnormals only, +-65504 beside subnormals, and scaled normal keys."""
    rng = np.random.default_rng(seed)
    k = np.zeros((T, H, D), dtype=np.uint16)
    for t in range(T):
        for h in range(H):
            kind = (t * H + h) % 8
            if kind == 0:
                continue
            if kind == 1:
                k[t, h, rng.integers(D)] = rng.integers(1, 0x7c00) | (rng.integers(2) << 15)
            elif kind == 2:
                e = rng.integers(0, 30)
                k[t, h, rng.choice(D, 4, replace=False)] = (e << 10) if e else 1 << rng.integers(10)
            elif kind == 3:
                k[t, h] = (rng.integers(0, 31, D) << 10) | rng.integers(0, 1024, D) | (rng.integers(0, 2, D) << 15)
            elif kind == 4:
                k[t, h] = rng.integers(0, 1024, D) | (rng.integers(0, 2, D) << 15)
            elif kind == 5:
                v = rng.integers(0, 1024, D) | (rng.integers(0, 2, D) << 15)
                v[rng.choice(D, 3, replace=False)] = 0x7bff | (rng.integers(2) << 15)
                k[t, h] = v
            else:
                x = rng.standard_normal(D) * 2.0 ** rng.integers(-20, 13)
                k[t, h] = np.clip(x, -65504, 65504).astype(np.float16).view(np.uint16)
    return k


@pytest.mark.parametrize("D", [64, 128])
def test_code_error_bit_exact_extreme_keys(D):
    """Key norms from zero to fp16 overflow range, over partial blocks: the
    errors bit-exact with the oracle's division by the norm."""
    cfg = small_workload(D=D, Hq=4, Hkv=2, S=1, T=600, seed=90 + D)
    case = make_case(cfg, lens=[600])
    keys = _extreme_keys(600, 2, D, seed=D)
    assert np.isfinite(keys.view(np.float16)).all()
    case["keys"] = torch.from_numpy(keys.view(np.float16))
    r, c8, c4 = _codes(case)
    rng = np.random.default_rng(D + 1)
    rc8 = rng.integers(0, 256, c8.shape).astype(np.uint8)
    rc4 = rng.integers(0, 256, c4.shape).astype(np.uint8)
    geom = geom_of(cfg)
    k = to_dev(case["keys"])
    cb8, cb4 = to_dev(case["cb8"]), to_dev(case["cb4"])
    for codes8, codes4, label in ((c8, c4, "nearest"), (rc8, rc4, "random")):
        flush(f"[code_error extreme keys] D={D} {label}")
        e8 = torch.full(c8.shape[:2], float("nan"), device="cuda")
        e4 = torch.full(c8.shape[:2], float("nan"), device="cuda")
        ada.code_error(geom, k, cb8, cb4, to_dev(codes8), to_dev(codes4), e8, e4)
        torch.cuda.synchronize()
        r8, r4 = oracle.code_error(case["keys"], case["cb8"], case["cb4"], codes8, codes4)
        assert np.isfinite(r8).all() and np.isfinite(r4).all()
        assert np.array_equal(e8.cpu().numpy(), r8) and np.array_equal(e4.cpu().numpy(), r4)

@pytest.mark.parametrize("D", [64, 128])
def test_code_error_bit_exact_codewords_on_the_key(D):
    """Codewords equal to the key's direction rounded to binary32, or one
    binary32 ulp from it: errors of about 1e-15 or exactly zero, which the
    kernel's fast form cannot round with certainty, so these states take
    the defined path (division rounded, each term rounded).  Bit-exact with
    the oracle over partial blocks (600 tokens)."""
    cfg = small_workload(D=D, Hq=4, Hkv=2, S=1, T=600, seed=95 + D)
    case = make_case(cfg, lens=[600])
    T, H, G = 600, 2, D // 8
    x = case["keys"].double().numpy()                       # [T][H][D]
    u = x / np.sqrt((x * x).sum(-1, keepdims=True))
    cb8 = case["cb8"].numpy().copy()                         # [H][G][256][8]
    cb4 = case["cb4"].numpy().copy()                         # [H][G][16][8]
    rng = np.random.default_rng(D + 7)
    for h in range(H):
        for t in range(256):                                 # tokens 0..255: own 8-bit codeword
            w = u[t, h].astype(np.float32).reshape(G, 8)
            if t % 3 == 1:                                   # one ulp off in one coordinate
                j = rng.integers(8)
                w[:, j] = np.nextafter(w[:, j], np.float32(np.inf))
            cb8[h, :, t] = w
        for t in range(16):                                  # tokens 0..15: own 4-bit codeword
            cb4[h, :, t] = u[t, h].astype(np.float32).reshape(G, 8)
    tok = np.arange(T)
    c8 = np.repeat((tok % 256).astype(np.uint8)[:, None, None], H, 1).repeat(G, 2)
    nib = (tok % 16).astype(np.uint8)
    c4 = np.repeat((nib | (nib << 4))[:, None, None], H, 1).repeat(G // 2, 2)
    geom = geom_of(cfg)
    flush(f"[code_error codewords on the key] D={D}")
    e8 = torch.full((T, H), float("nan"), device="cuda")
    e4 = torch.full((T, H), float("nan"), device="cuda")
    ada.code_error(geom, to_dev(case["keys"]), to_dev(torch.from_numpy(cb8)), to_dev(torch.from_numpy(cb4)),
                   to_dev(c8), to_dev(c4), e8, e4)
    torch.cuda.synchronize()
    r8, r4 = oracle.code_error(case["keys"], torch.from_numpy(cb8), torch.from_numpy(cb4), c8, c4)
    assert (r8[:256] < 1e-12).all() and (r4[:16] < 1e-12).all()   # the cases are the tiny errors
    assert np.array_equal(e8.cpu().numpy(), r8) and np.array_equal(e4.cpu().numpy(), r4)


def _solve_both(geom, D, cu, budgets, r, e8, e4, sc, prot=None):
    tiers = torch.full(r.shape, 77, dtype=torch.uint8, device="cuda")
    ada.rdr_solve(geom, cu, budgets, to_dev(r), to_dev(e8), to_dev(e4), to_dev(sc), tiers,
                  protect=None if prot is None else to_dev(prot))
    torch.cuda.synchronize()
    ref = oracle.rdr_solve(D, cu, budgets, r, e8, e4, sc, protect=prot)
    return tiers.cpu().numpy(), ref


def test_rdr_solve_golden_hand_cases():
    with open(os.path.join(GOLDEN, "rdr_solve_hand.json")) as f:
        g = json.load(f)
    st = g["states"]
    n = len(st)
    geom = ada.Geom(g["D"], 1, 1)
    r = np.array([[x["radius"]] for x in st], np.float16).view(np.uint16)
    e8 = np.array([[x["err8"]] for x in st], np.float32)
    e4 = np.array([[x["err4"]] for x in st], np.float32)
    sc = np.array([[x["score"]] for x in st], np.float32)
    reserve = 15 * (256 + 144 + 72)
    for case in g["cases"]:
        pr = None if "protect" not in case else np.array(case["protect"], np.uint8).reshape(n, 1)
        got, ref = _solve_both(geom, g["D"], [0, n], [case["cap"] + reserve], r, e8, e4, sc, pr)
        assert got.ravel().tolist() == case["tiers"] == ref.ravel().tolist(), case["note"]


@pytest.mark.parametrize("D,H", [(128, 8), (64, 4), (128, 1)])
def test_rdr_solve_bit_exact_ragged(D, H):
    """Several sequences (one empty, one of a single token, others spanning
    several 1024-state blocks with ragged ends), budgets from infeasible to
    non-binding, with and without protection."""
    rng = np.random.default_rng(D + H)
    lens = [700, 0, 1, 2100, 333, 64]
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    r = (rng.lognormal(2.0, 0.6, (N, H)).astype(np.float16)).view(np.uint16)
    e8 = rng.uniform(0.05, 0.5, (N, H)).astype(np.float32)
    e4 = (e8 + rng.uniform(-0.05, 0.5, (N, H))).clip(0, 2).astype(np.float32)
    sc = np.minimum(rng.zipf(1.1, (N, H)), 1 << 24).astype(np.float32)
    sc[rng.random((N, H)) < 0.01] = 0.0           # zero utility: free to drop
    prot = (rng.random((N, H)) < 0.02).astype(np.uint8)
    R0 = ada.page_bytes(D, 0) // 16
    dense = np.array(lens, np.int64) * H * R0
    geom = ada.Geom(D, H, H)
    for frac in (0.0, 0.1, 0.35, 0.6, 0.9, 1.2):
        budgets = (dense * frac).astype(np.int64)
        for pr in (None, prot):
            flush(f"[solve] D={D} H={H} budget {frac} protect={pr is not None}")
            got, ref = _solve_both(geom, D, cu, budgets, r, e8, e4, sc, pr)
            assert np.array_equal(got, ref), int((got != ref).sum())


def test_tier_counts_and_pack_tiers_bit_exact_then_decode():
    cfg = small_workload(D=128, Hq=8, Hkv=2, S=3, T=900, seed=90)
    lens = [900, 250, 17]
    case = make_case(cfg, lens=lens)
    geom = geom_of(cfg)
    r, c8, c4 = _codes(case)
    e8, e4 = oracle.code_error(case["keys"], case["cb8"], case["cb4"], c8, c4)
    budgets = synth.budget_bytes(cfg, lens) * 5 // 6
    tiers = oracle.rdr_solve(128, case["cu"], budgets, r, e8, e4, case["scores"].numpy())
    counts = oracle.row_tier_counts(case["cu"], tiers)
    flush("[tier_counts]")
    got = ada.tier_counts(geom, case["cu"], to_dev(tiers))
    assert np.array_equal(got, counts)
    n_pages = ada.pack_tiers_num_pages(geom, counts)
    perm = np.random.default_rng(5).permutation(n_pages).astype(np.uint32)
    maxp = max(lens) // 16 + 4
    arena = int(sum(lens) * 2 * 512 + 3 * 2 * 3 * 8192)
    hc = oracle.HostCache(128, 2, 3, maxp, arena)
    assert oracle.pack_tiers(hc, case["cu"], tiers, case["keys"], case["values"], r, c8, c4,
                             place_perm=perm) == 0
    flush("[pack_tiers]")
    dc = ada.Cache(geom, 3, maxp, arena, slot_tokens=True)
    ada.rdr_pack_tiers(geom, dc, case["cu"], got, to_dev(tiers), to_dev(case["keys"]),
                       to_dev(case["values"]), to_dev(r), to_dev(c8), to_dev(c4), place_perm=perm)
    torch.cuda.synchronize()
    assert int(dc.cursor[0]) == int(hc.cursor[0])
    used = int(hc.cursor[0]) * 128
    assert np.array_equal(dc.arena[:used].cpu().numpy(), hc.arena[:used])
    assert np.array_equal(dc.page_table.cpu().numpy().view(np.uint32), hc.page_table)
    assert np.array_equal(dc.page_meta.cpu().numpy(), hc.page_meta)
    assert np.array_equal(dc.num_pages.cpu().numpy(), hc.num_pages)
    assert np.array_equal(dc.tier_tokens.cpu().numpy(), hc.tier_tokens)
    assert np.array_equal(dc.slot_token.cpu().numpy(), hc.slot_token)
    assert np.array_equal(dc.num_pages_host, hc.num_pages)
    # the stored bytes stay within each sequence's budget
    for s in range(3):
        rows = slice(2 * s, 2 * s + 2)
        b = sum(oracle.page_bytes(128, k) * -(-int(c) // 16) for row in counts[rows] for k, c in enumerate(row))
        assert b <= budgets[s]
    flush("[decode of the solver-built cache]")
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, nthreads=8)
    out, lse, _ = decode_outputs(geom, dc, to_dev(case["q"]), with_logits=False)
    ada.decode(geom, dc, to_dev(case["cb8"]), to_dev(case["cb4"]), to_dev(case["q"]), cfg.sigma, out, lse)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().double().numpy() - ref["out"]).max() <= OUT_TOL
    l = lse.cpu().double().numpy()
    fin = np.isfinite(ref["lse"])  # a row left with no pages has lse = -inf
    assert np.array_equal(np.isfinite(l), fin) and (l[~fin] == -np.inf).all()
    assert (np.abs(l[fin] - ref["lse"][fin]) <= 1e-3 * np.maximum(np.abs(ref["lse"][fin]), 1.0)).all()


def test_gpu_encode_error_solve_chain_matches_oracle():
    """The append path on the GPU (encode -> code error -> solve -> counts)
    equals the oracle's on the same keys and codes, bit for bit."""
    cfg = small_workload(D=64, Hq=8, Hkv=4, S=2, T=1500, seed=91)
    lens = [1500, 611]
    case = make_case(cfg, lens=lens)
    geom = geom_of(cfg)
    k = to_dev(case["keys"])
    cb8, cb4 = to_dev(case["cb8"]), to_dev(case["cb4"])
    flush("[chain] encode + code error + solve on the GPU")
    r, c8, c4 = gpu_encode(geom, k, cb8, cb4)
    e8 = torch.empty(r.shape, device="cuda")
    e4 = torch.empty(r.shape, device="cuda")
    ada.code_error(geom, k, cb8, cb4, c8, c4, e8, e4)
    budgets = synth.budget_bytes(cfg, lens) // 2
    tiers = torch.empty(r.shape, dtype=torch.uint8, device="cuda")
    ada.rdr_solve(geom, case["cu"], budgets, r, e8, e4, to_dev(case["scores"]), tiers)
    counts = ada.tier_counts(geom, case["cu"], tiers)
    # (the oracle takes the GPU's codes: encode parity is tested on its own)
    rr, rc8, rc4 = u16(r), c8.cpu().numpy(), c4.cpu().numpy()
    re8, re4 = oracle.code_error(case["keys"], case["cb8"], case["cb4"], rc8, rc4)
    assert np.array_equal(e8.cpu().numpy(), re8) and np.array_equal(e4.cpu().numpy(), re4)
    rt = oracle.rdr_solve(64, case["cu"], budgets, rr, re8, re4, case["scores"].numpy())
    assert np.array_equal(tiers.cpu().numpy(), rt)
    assert np.array_equal(counts, oracle.row_tier_counts(case["cu"], rt))


def _row_contents(meta, pt, arena, npg, tt, slots, row, D):
    """A row's pages (metadata, bytes, slot positions) and counts, found
    through its own page table: placement-independent."""
    out = []
    for p in range(int(npg[row])):
        m = int(meta[row, p])
        off = int(pt[row, p]) * 128
        out.append((m, arena[off:off + oracle.page_bytes(D, m & 3)].tobytes(),
                    tuple(slots[row, p]) if slots is not None else None))
    return out, tuple(int(x) for x in tt[row])


@pytest.mark.parametrize("D,H", [(128, 2), (64, 4)])
def test_pack_tiers_device_equals_the_host_planned_pack(D, H):
    """The device-planned pack (rows take arena blocks from a device cursor)
    holds, row by row, exactly the pages rdr_pack_tiers / the oracle's
    pack_tiers build from the same tiers; two calls in a row append; the
    pool is tiled by the rows' blocks; then decode matches the oracle."""
    cfg = small_workload(D=D, Hq=2 * H, Hkv=H, S=3, T=900, seed=92 + D)
    lens = [900, 250, 17]
    case = make_case(cfg, lens=lens)
    geom = geom_of(cfg)
    r, c8, c4 = _codes(case)
    e8, e4 = oracle.code_error(case["keys"], case["cb8"], case["cb4"], c8, c4)
    budgets = synth.budget_bytes(cfg, lens) * 5 // 6
    tiers = oracle.rdr_solve(D, case["cu"], budgets, r, e8, e4, case["scores"].numpy())
    # two calls: the first 60% of each sequence's tokens, then the rest
    cut = [int(0.6 * T) for T in lens]
    parts = []
    for lo, hi in (([0, 0, 0], cut), (cut, lens)):
        idx = np.concatenate([np.arange(int(case["cu"][s]) + lo[s], int(case["cu"][s]) + hi[s]) for s in range(3)])
        cu = synth.cu_tokens([hi[s] - lo[s] for s in range(3)])
        parts.append((idx, cu, list(lo)))
    maxp = max(lens) // 16 + 8
    arena = int(sum(lens) * H * 512 + 3 * H * 6 * 8192)
    hc = oracle.HostCache(D, H, 3, maxp, arena)
    dc = ada.Cache(geom, 3, maxp, arena, slot_tokens=True)
    state = ada.AppendState(geom, dc)
    for idx, cu, pos in parts:
        t = tiers[idx]
        assert oracle.pack_tiers(hc, cu, t, case["keys"][idx], case["values"][idx], r[idx], c8[idx], c4[idx],
                                 pos_base=np.array(pos, np.int64)) == 0
        flush(f"[pack_tiers_device] D={D} H={H}: {len(idx)} tokens")
        ada.rdr_pack_tiers_device(geom, dc, state, cu, to_dev(t), to_dev(case["keys"][idx]),
                                  to_dev(case["values"][idx]), to_dev(r[idx]), to_dev(c8[idx]), to_dev(c4[idx]),
                                  pos_base=np.array(pos, np.int64))
    assert state.pull() == 0
    assert int(dc.cursor[0]) == int(hc.cursor[0])
    g_meta, g_pt = dc.page_meta.cpu().numpy(), dc.page_table.cpu().numpy().view(np.uint32)
    g_ar, g_np = dc.arena.cpu().numpy(), dc.num_pages.cpu().numpy()
    g_tt, g_sl = dc.tier_tokens.cpu().numpy(), dc.slot_token.cpu().numpy()
    assert np.array_equal(g_np[:3 * H], hc.num_pages)
    for row in range(3 * H):
        assert _row_contents(g_meta, g_pt, g_ar, g_np, g_tt, g_sl, row, D) == \
            _row_contents(hc.page_meta, hc.page_table, hc.arena, hc.num_pages, hc.tier_tokens, hc.slot_token, row, D)
    # the rows' blocks tile the pool from 0 to the cursor
    offs, ends = [], []
    for row in range(3 * H):
        for p in range(int(g_np[row])):
            o = int(g_pt[row, p])
            offs.append(o)
            ends.append(o + oracle.page_bytes(D, int(g_meta[row, p]) & 3) // 128)
    order = np.argsort(offs)
    o, e = np.array(offs)[order], np.array(ends)[order]
    assert o[0] == 0 and np.array_equal(o[1:], e[:-1]) and e[-1] == int(dc.cursor[0])
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, nthreads=8)
    out, lse, _ = decode_outputs(geom, dc, to_dev(case["q"]), with_logits=False)
    ada.decode(geom, dc, to_dev(case["cb8"]), to_dev(case["cb4"]), to_dev(case["q"]), cfg.sigma, out, lse)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().double().numpy() - ref["out"]).max() <= OUT_TOL


def test_pack_tiers_device_capacity_status_bits():
    """A row whose pages pass max_pages_per_head, or whose block passes the
    arena, stores nothing and sets its status bit; the other rows are
    packed as usual."""
    cfg = small_workload(D=64, Hq=2, Hkv=2, S=1, T=100, seed=95)
    case = make_case(cfg, lens=[100])
    geom = geom_of(cfg)
    r, c8, c4 = _codes(case)
    tiers = np.zeros((100, 2), np.uint8)
    tiers[:, 1] = 3            # head 1 drops everything: no pages
    args = (to_dev(tiers), to_dev(case["keys"]), to_dev(case["values"]), to_dev(r), to_dev(c8), to_dev(c4))
    dc = ada.Cache(geom, 1, 4, 1 << 20)    # 7 fp16 pages needed, room for 4
    st = ada.AppendState(geom, dc)
    ada.rdr_pack_tiers_device(geom, dc, st, case["cu"], *args)
    assert st.pull() == 1 and int(dc.num_pages[0]) == 0 and int(dc.cursor[0]) == 0
    dc = ada.Cache(geom, 1, 16, 6 * 4096)  # room for 6 of the 7 fp16 pages
    st = ada.AppendState(geom, dc)
    ada.rdr_pack_tiers_device(geom, dc, st, case["cu"], *args)
    assert st.pull() == 2 and int(dc.num_pages[0]) == 0 and int(dc.cursor[0]) == 0
    dc = ada.Cache(geom, 1, 16, 7 * 4096)  # exactly enough
    st = ada.AppendState(geom, dc)
    ada.rdr_pack_tiers_device(geom, dc, st, case["cu"], *args)
    assert st.pull() == 0 and int(dc.num_pages[0]) == 7 and int(dc.cursor[0]) == 7 * 32
