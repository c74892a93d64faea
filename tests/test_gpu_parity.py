"""GPU parity: the HIP library through its C ABI against the CPU oracle on the
same seeded inputs.

Bars (written here, from the method's targets): encode codes and radii
bit-exact (both sides give the double-precision argmin: the kernel's
binary32 filter decides only where its error bound proves the winner, and
rescans in double otherwise); pages, page tables, metadata and tier
counts bit-exact when both packs get the same encode outputs; logits within
|d| <= 1e-3 * max(|l|, 1e-2); outputs max-abs <= 1e-2 (fp32 accumulation);
lse within 1e-3 * max(|lse|, 1)."""
import numpy as np
import pytest
import torch

import compressed_kv_attention_amd as ada
import oracle
import synth
from gpu_util import (decode_outputs, flush, geom_of, gpu_encode, logit_tol_ok, to_dev, u16,
                      upload_cache)
from helpers import make_case, oracle_cache, small_workload

pytestmark = pytest.mark.gpu

OUT_TOL = 1e-2


def _dev_case(case):
    return {k: to_dev(case[k]) for k in ("keys", "values", "scores", "q", "cb8", "cb4")}


def _check_decode(geom, hc, case, num_splits=0, label=""):
    flush(f"[decode] {label} splits={num_splits}")
    cfg = case["cfg"]
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True, nthreads=8)
    dc = upload_cache(hc, geom)
    d = _dev_case(case)
    out, lse, lg = decode_outputs(geom, dc, d["q"])
    ada.decode(geom, dc, d["cb8"], d["cb4"], d["q"], cfg.sigma, out, lse, lg, num_splits=num_splits)
    torch.cuda.synchronize()
    ok, worst = logit_tol_ok(lg.cpu().double().numpy(), ref["logits"])
    assert ok, f"logits off by {worst:.3g} (relative)"
    o = out.cpu().double().numpy()
    err = np.abs(o - ref["out"]).max(initial=0.0)
    assert err <= OUT_TOL, f"out max-abs {err:.3g}"
    l = lse.cpu().double().numpy()
    fin = np.isfinite(ref["lse"])
    assert np.array_equal(np.isfinite(l), fin)
    assert (np.abs(l[fin] - ref["lse"][fin]) <= 1e-3 * np.maximum(np.abs(ref["lse"][fin]), 1.0)).all()
    assert (l[~fin] == -np.inf).all() and not o[~fin].any()
    flush(f"[decode] {label} ok: out max-abs {err:.2e}, logits rel {worst:.2e}")
    return err


@pytest.mark.parametrize("splits", [0, 1, 3])
def test_decode_tiny_workload(splits):
    cfg = synth.WORKLOADS[1]
    case = make_case(cfg)
    hc, _ = oracle_cache(case)
    _check_decode(geom_of(cfg), hc, case, splits, "tiny D=64 MHA T=512")


@pytest.mark.parametrize("splits", [1, 4])
def test_decode_stages_equal_one_call(splits):
    """ada_decode_stream + ada_decode_merge on one stream give exactly the
    outputs of one ada_decode call (same kernels, same order)."""
    cfg = small_workload(D=128, Hq=8, Hkv=2, S=3, T=700, seed=61)
    case = make_case(cfg, lens=[700, 333, 90], mixes=[(1500, 6000, 8500)] * 3)
    hc, _ = oracle_cache(case)
    geom = geom_of(cfg)
    dc = upload_cache(hc, geom)
    d = _dev_case(case)
    flush(f"[stages] splits={splits}")
    out1, lse1, lg1 = decode_outputs(geom, dc, d["q"])
    ada.decode(geom, dc, d["cb8"], d["cb4"], d["q"], cfg.sigma, out1, lse1, lg1, num_splits=splits)
    out2, lse2, lg2 = decode_outputs(geom, dc, d["q"])
    ws = None
    for st in ("stream", "merge"):
        ws = ada.decode_stage(st, geom, dc, d["cb8"], d["cb4"], d["q"], cfg.sigma, out2, lse2, lg2,
                              num_splits=splits, ws=ws)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    assert torch.equal(torch.nan_to_num(lg1, nan=7.0), torch.nan_to_num(lg2, nan=7.0))
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, nthreads=8)
    assert np.abs(out2.cpu().double().numpy() - ref["out"]).max() <= OUT_TOL


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 4, 2), (64, 8, 2), (128, 4, 4), (64, 2, 2),
                                     (128, 10, 2), (64, 5, 1), (128, 16, 2), (64, 16, 2),
                                     (64, 4, 2)])
def test_decode_ragged_mixed_tiers(D, Hq, Hkv):
    cfg = small_workload(D=D, Hq=Hq, Hkv=Hkv, S=4, T=300, seed=40 + D + Hq)
    mixes = [(1500, 6000, 8500), (0, 0, 0), (10000, 10000, 10000), (0, 3000, 9000)]
    case = make_case(cfg, lens=[300, 40, 17, 0], mixes=mixes)
    hc, _ = oracle_cache(case)
    for sp in (0, 1, 5):
        _check_decode(geom_of(cfg), hc, case, sp, f"ragged D={D} Hq={Hq} Hkv={Hkv}")


@pytest.mark.parametrize("D,ratio", [(128, 5), (128, 8), (64, 8), (128, 4)])
def test_decode_growing_logits_rescale_per_head(D, ratio):
    """Keys grow along the sequence and each query head has its own scale,
    so the running maxima of the heads of one group jump on different pages
    (the rescale of one head must leave the others' accumulators alone)."""
    cfg = small_workload(D=D, Hq=2 * ratio, Hkv=2, S=2, T=900, seed=70 + D + ratio)
    case = make_case(cfg, lens=[900, 411], mixes=[(2000, 6000, 9000)] * 2)
    N = case["N"]
    grow = (1.0 + torch.arange(N, dtype=torch.float32) / 60.0).view(N, 1, 1)
    case["keys"] = (case["keys"].float() * grow).to(torch.float16)
    hs = (1.0 + 0.7 * torch.arange(cfg.num_q_heads, dtype=torch.float32)).view(1, -1, 1)
    case["q"] = (case["q"].float() * hs).to(torch.bfloat16)
    hc, _ = oracle_cache(case)
    for sp in (1, 3):
        _check_decode(geom_of(cfg), hc, case, sp, f"growing logits D={D} GQA {ratio}")


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (64, 4, 4), (128, 10, 2), (64, 16, 2),
                                     (128, 4, 2), (64, 4, 2), (128, 16, 2), (64, 10, 2), (128, 3, 3)])
def test_decode_sym_matches_oracle(D, Hq, Hkv):
    """The symmetric angle-code variant (query codes) against the oracle's:
    logits to the decode bar (so the query codes agree), outputs, lse."""
    cfg = small_workload(D=D, Hq=Hq, Hkv=Hkv, S=3, T=400, seed=95 + D + Hq)
    case = make_case(cfg, lens=[400, 77, 0], mixes=[(1500, 6000, 8500), (0, 5000, 10000), (0, 0, 0)])
    hc, _ = oracle_cache(case)
    geom = geom_of(cfg)
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True, nthreads=8, sym=True)
    dc = upload_cache(hc, geom)
    d = _dev_case(case)
    for sp in (0, 1, 3):
        flush(f"[decode_sym] D={D} Hq={Hq} Hkv={Hkv} splits={sp}")
        out, lse, lg = decode_outputs(geom, dc, d["q"])
        ada.decode_sym(geom, dc, d["cb8"], d["cb4"], d["q"], cfg.sigma, out, lse, lg, num_splits=sp)
        torch.cuda.synchronize()
        ok, worst = logit_tol_ok(lg.cpu().double().numpy(), ref["logits"])
        assert ok, f"logits off by {worst:.3g} (relative)"
        o = out.cpu().double().numpy()
        assert np.abs(o - ref["out"]).max(initial=0.0) <= OUT_TOL
        l = lse.cpu().double().numpy()
        fin = np.isfinite(ref["lse"])
        assert np.array_equal(np.isfinite(l), fin)
        assert (np.abs(l[fin] - ref["lse"][fin]) <= 1e-3 * np.maximum(np.abs(ref["lse"][fin]), 1.0)).all()
    # the variant really differs from the asymmetric decode on coded slots
    asym = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True)
    m = ~np.isnan(ref["logits"])
    assert np.abs(asym["logits"][m] - ref["logits"][m]).max() > 1e-2


@pytest.mark.parametrize("mix", [(10000, 10000, 10000), (0, 10000, 10000), (0, 0, 10000)])
def test_decode_single_token_rows(mix):
    cfg = small_workload(D=128, Hq=4, Hkv=1, S=3, T=1, mix=mix, seed=50)
    case = make_case(cfg, lens=[1, 1, 1])
    hc, _ = oracle_cache(case)
    _check_decode(geom_of(cfg), hc, case, 0, f"single token {mix}")


def test_decode_permuted_pool_and_appends():
    cfg = small_workload(D=128, Hq=8, Hkv=2, S=2, T=200, seed=51)
    case = make_case(cfg, lens=[200, 150, 64, 33], mixes=[(1000, 5000, 8000)] * 4)
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    hc = oracle.HostCache(128, 2, 2, 64, 4 << 20)
    cu1, cu2 = np.array([0, 200, 350], np.int32), np.array([0, 64, 97], np.int32)
    bp = np.array([(1000, 5000, 8000)] * 2, np.int32)
    n1 = oracle.num_pages_of_call(128, 2, cu1, bp)
    perm = np.random.default_rng(3).permutation(n1).astype(np.uint32)
    assert oracle.pack(hc, cu1, bp, case["keys"][:350], case["values"][:350], r[:350], c8[:350],
                       c4[:350], case["scores"][:350], place_perm=perm) == 0
    assert oracle.pack(hc, cu2, bp, case["keys"][350:], case["values"][350:], r[350:], c8[350:],
                       c4[350:], case["scores"][350:], pos_base=[200, 150]) == 0
    _check_decode(geom_of(cfg), hc, case, 0, "permuted pool + append")
    _check_decode(geom_of(cfg), hc, case, 2, "permuted pool + append")


def test_decode_llama_shape_t32k_full():
    cfg = synth.WORKLOADS[2]
    case = make_case(cfg)
    hc, _ = oracle_cache(case, maxp=1760)
    for sp in (0, 7):
        _check_decode(geom_of(cfg), hc, case, sp, "Llama-3-8B shape T=32768")


# ---- encode ---------------------------------------------------------------

def _check_encode(cfg, case, label):
    flush(f"[encode] {label}")
    geom = geom_of(cfg)
    d = _dev_case(case)
    r, c8, c4 = gpu_encode(geom, d["keys"], d["cb8"], d["cb4"])
    torch.cuda.synchronize()
    rr, rc8, rc4 = oracle.encode(case["keys"], case["cb8"], case["cb4"], nthreads=8)
    assert np.array_equal(u16(r), rr), "radius differs"
    g8, g4 = c8.cpu().numpy(), c4.cpu().numpy()
    agree8 = (g8 == rc8).mean()
    agree4 = (g4 == rc4).mean()
    flush(f"[encode] {label}: codes8 agree {agree8:.6f}, codes4 agree {agree4:.6f}")
    assert agree8 == 1.0 and agree4 == 1.0
    return r, c8, c4


def test_encode_tiny_and_small():
    _check_encode(synth.WORKLOADS[1], make_case(synth.WORKLOADS[1]), "tiny")
    cfg = small_workload(D=128, Hq=4, Hkv=2, S=2, T=333, seed=60)
    case = make_case(cfg)
    # a zero key and a key of one huge channel
    case["keys"][5, 0] = 0
    case["keys"][7, 1] = 0
    case["keys"][7, 1, 3] = 60000.0
    _check_encode(cfg, case, "D=128 with zero and extreme keys")



def test_encode_radius_at_fp16_rounding_boundaries():
    """Keys whose norm is an fp16 rounding midpoint exactly, or just above
    one: 2^k (1, 2^-5, 2^-11) has norm 2^k (1 + 2^-11), the midpoint between
    2^k and its fp16 successor (a tie: rounds to even), and a fourth
    coordinate of 2^(k-24) moves it above the midpoint by 2^-49 relative
    (rounds up).  The radius must follow the defining norm bit for bit."""
    cfg = small_workload(D=128, Hq=4, Hkv=2, S=1, T=96, seed=63)
    case = make_case(cfg)
    k = case["keys"]
    for t in range(96):
        for hh in range(2):
            e = (t % 24) - 8 if hh == 0 else (t % 16)
            row = torch.zeros(128, dtype=torch.float32)
            row[[3, 40, 77]] = torch.tensor([2.0 ** e, 2.0 ** (e - 5), 2.0 ** (e - 11)])
            if t % 2 and e - 24 >= -24:
                row[120] = 2.0 ** (e - 24)
            k[t, hh] = row.to(torch.float16)
    assert torch.isfinite(k.float()).all()
    _check_encode(cfg, case, "norms at fp16 rounding midpoints")

def test_encode_near_ties_exact():
    """Codebooks whose codewords come in pairs -- equal, or one binary32 ulp
    apart in one coordinate -- make nearly every nearest codeword a near tie
    that binary32 scores cannot separate; the codes must still equal the
    double-precision argmin (lowest index on an exact tie) bit for bit."""
    cfg = small_workload(D=64, Hq=4, Hkv=2, S=2, T=300, seed=61)
    case = make_case(cfg)
    for name in ("cb8", "cb4"):
        cb = case[name].numpy().copy()
        odd = cb[..., 0::2, :].copy()
        odd[..., 0::2, 3] = np.nextafter(odd[..., 0::2, 3], np.float32(np.inf))
        cb[..., 1::2, :] = odd
        case[name] = torch.from_numpy(cb)
    flush("[encode] paired codewords")
    geom = geom_of(cfg)
    d = _dev_case(case)
    r, c8, c4 = gpu_encode(geom, d["keys"], d["cb8"], d["cb4"])
    torch.cuda.synchronize()
    rr, rc8, rc4 = oracle.encode(case["keys"], case["cb8"], case["cb4"], nthreads=8)
    assert np.array_equal(u16(r), rr)
    assert np.array_equal(c8.cpu().numpy(), rc8)
    assert np.array_equal(c4.cpu().numpy(), rc4)


def test_encode_codebooks_outside_the_filter_range():
    """Codebooks the binary32 filter cannot bound -- a group with entries of
    magnitude 2^30, a group with a NaN codeword, a group with an infinite
    entry -- are scanned in double for every token (a NaN or infinite
    distance never wins); the other groups keep the filter.  Codes equal the
    oracle's bit for bit."""
    cfg = small_workload(D=64, Hq=4, Hkv=2, S=1, T=200, seed=62)
    case = make_case(cfg)
    cb8 = case["cb8"].numpy().copy()
    cb4 = case["cb4"].numpy().copy()
    cb8[0, 1] *= np.float32(2.0 ** 30)        # head 0, group 1: far outside
    cb8[1, 3, 7, :] = np.float32(np.nan)      # head 1, group 3: a NaN codeword
    cb4[1, 5, 2, 0] = np.float32(np.inf)      # head 1, group 5: an infinite entry
    case["cb8"], case["cb4"] = torch.from_numpy(cb8), torch.from_numpy(cb4)
    flush("[encode] codebooks outside the filter range")
    geom = geom_of(cfg)
    d = _dev_case(case)
    r, c8, c4 = gpu_encode(geom, d["keys"], d["cb8"], d["cb4"])
    torch.cuda.synchronize()
    rr, rc8, rc4 = oracle.encode(case["keys"], case["cb8"], case["cb4"], nthreads=8)
    assert np.array_equal(u16(r), rr)
    assert np.array_equal(c8.cpu().numpy(), rc8)
    assert np.array_equal(c4.cpu().numpy(), rc4)


def test_encode_llama_shape_t32k_full():
    cfg = synth.WORKLOADS[2]
    _check_encode(cfg, make_case(cfg), "Llama-3-8B shape T=32768")


# ---- pack -----------------------------------------------------------------

def _gpu_pack_like(hc_ref, geom, calls, slot_tokens=True):
    """Replays oracle pack calls on the GPU; returns the device cache."""
    dc = ada.Cache(geom, hc_ref.S, hc_ref.maxp, len(hc_ref.arena), slot_tokens=slot_tokens)
    for c in calls:
        ada.rdr_pack(geom, dc, c["cu"], c["bp"], to_dev(c["keys"]), to_dev(c["values"]),
                     to_dev(c["radius"]), to_dev(c["codes8"]), to_dev(c["codes4"]),
                     to_dev(c["scores"]), protect=c.get("protect"), place_perm=c.get("perm"),
                     pos_base=c.get("pos_base"))
    torch.cuda.synchronize()
    return dc


def _compare_caches(dc, hc, label):
    used = int(hc.cursor[0]) * 128
    assert int(dc.cursor[0]) == int(hc.cursor[0]), label
    assert np.array_equal(dc.num_pages_host[: len(hc.num_pages)], hc.num_pages)
    a = dc.arena[:used].cpu().numpy()
    diff = np.nonzero(a != hc.arena[:used])[0]
    assert len(diff) == 0, f"{label}: {len(diff)} arena bytes differ, first at {diff[:5]}"
    rows = len(hc.num_pages)
    assert np.array_equal(dc.num_pages[:rows].cpu().numpy(), hc.num_pages)
    assert np.array_equal(dc.tier_tokens[:rows].cpu().numpy(), hc.tier_tokens)
    for r in range(rows):
        n = hc.num_pages[r]
        assert np.array_equal(dc.page_table[r, :n].cpu().numpy().view(np.uint32), hc.page_table[r, :n])
        assert np.array_equal(dc.page_meta[r, :n].cpu().numpy(), hc.page_meta[r, :n])
        if dc.slot_token is not None:
            assert np.array_equal(dc.slot_token[r, :n].cpu().numpy(), hc.slot_token[r, :n])


def test_pack_tiny_bit_exact():
    cfg = synth.WORKLOADS[1]
    case = make_case(cfg)
    flush("[pack] tiny")
    hc, (r, c8, c4) = oracle_cache(case)
    dc = _gpu_pack_like(hc, geom_of(cfg), [dict(cu=case["cu"], bp=case["bp"], keys=case["keys"],
                                                values=case["values"], radius=r, codes8=c8, codes4=c4,
                                                scores=case["scores"])])
    _compare_caches(dc, hc, "tiny")


@pytest.mark.parametrize("D", [64, 128])
def test_pack_ragged_protect_permuted_two_calls(D):
    cfg = small_workload(D=D, Hq=4, Hkv=2, S=3, T=100, seed=70 + D)
    lens = np.array([500, 37, 0, 20, 0, 45])
    case = make_case(cfg, lens=lens, mixes=[(2500, 7500, 9000)] * 6)
    flush(f"[pack] ragged D={D}")
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    rng = np.random.default_rng(D)
    scores = torch.from_numpy(rng.integers(1, 5, (case["N"], 2)).astype(np.float32))
    scores[3, 0] = -0.0  # signed zero ties with +0
    scores[4, 0] = 0.0
    N1 = 537
    cu1, cu2 = np.array([0, 500, 537, 537], np.int32), np.array([0, 20, 20, 65], np.int32)
    bp1 = np.array([(2500, 7500, 9000), (1000, 5000, 10000), (3000, 3000, 3000)], np.int32)
    bp2 = np.array([(10000, 10000, 10000), (5000, 5000, 5000), (0, 2000, 6000)], np.int32)
    protect = np.zeros((case["N"], 2), np.uint8)
    protect[[1, 9, 77, 300], 0] = 1
    protect[[2, 499], 1] = 1
    protect[500, 1] = 1
    hc = oracle.HostCache(D, 2, 3, 64, 2 << 20)
    n1 = oracle.num_pages_of_call(D, 2, cu1, bp1)
    perm1 = rng.permutation(n1).astype(np.uint32)
    calls = [dict(cu=cu1, bp=bp1, keys=case["keys"][:N1], values=case["values"][:N1], radius=r[:N1],
                  codes8=c8[:N1], codes4=c4[:N1], scores=scores[:N1], protect=protect[:N1], perm=perm1),
             dict(cu=cu2, bp=bp2, keys=case["keys"][N1:], values=case["values"][N1:], radius=r[N1:],
                  codes8=c8[N1:], codes4=c4[N1:], scores=scores[N1:],
                  pos_base=np.array([500, 37, 0], np.int64))]
    for c in calls:
        rc = oracle.pack(hc, c["cu"], c["bp"], c["keys"], c["values"], c["radius"], c["codes8"],
                         c["codes4"], c["scores"], protect=c.get("protect"), place_perm=c.get("perm"),
                         pos_base=c.get("pos_base"))
        assert rc == 0
    dc = _gpu_pack_like(hc, geom_of(cfg), calls)
    _compare_caches(dc, hc, f"ragged D={D}")


@pytest.mark.parametrize("D", [64, 128])
def test_pack_arena_order_page_list_equals_host_built_identity_order(D):
    """In arena order the page list is written on the device from the rows'
    entries; with the identity permutation the host builds it.  Both give
    the oracle's cache, over two calls (the second appends to every row)."""
    cfg = small_workload(D=D, Hq=16, Hkv=8, S=3, T=100, seed=90 + D)
    lens = np.array([333, 17, 0, 45, 160, 1])
    case = make_case(cfg, lens=lens, mixes=[(2000, 6000, 9000), (0, 10000, 10000), (5000, 5000, 5000),
                                            (10000, 10000, 10000), (0, 0, 6000), (0, 3000, 10000)])
    flush(f"[pack] arena-order page list D={D}")
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    N1 = 350
    cu1, cu2 = np.array([0, 333, 350, 350], np.int32), np.array([0, 45, 205, 206], np.int32)
    calls = [dict(cu=cu1, bp=case["bp"][:3], keys=case["keys"][:N1], values=case["values"][:N1], radius=r[:N1],
                  codes8=c8[:N1], codes4=c4[:N1], scores=case["scores"][:N1]),
             dict(cu=cu2, bp=case["bp"][3:], keys=case["keys"][N1:], values=case["values"][N1:], radius=r[N1:],
                  codes8=c8[N1:], codes4=c4[N1:], scores=case["scores"][N1:],
                  pos_base=np.array([333, 17, 0], np.int64))]
    hc = oracle.HostCache(D, 8, 3, 64, 4 << 20)
    for c in calls:
        assert oracle.pack(hc, c["cu"], c["bp"], c["keys"], c["values"], c["radius"], c["codes8"], c["codes4"],
                           c["scores"], pos_base=c.get("pos_base")) == 0
    geom = geom_of(cfg)
    _compare_caches(_gpu_pack_like(hc, geom, calls), hc, f"device page list D={D}")
    ident = []
    for c in calls:
        n = oracle.num_pages_of_call(D, 8, c["cu"], c["bp"])
        ident.append(dict(c, perm=np.arange(n, dtype=np.uint32)))
    _compare_caches(_gpu_pack_like(hc, geom, ident), hc, f"host page list D={D}")


def test_pack_llama_shape_t32k_full():
    cfg = synth.WORKLOADS[2]
    case = make_case(cfg)
    flush("[pack] Llama-3-8B shape T=32768")
    hc, (r, c8, c4) = oracle_cache(case, maxp=1760)
    dc = _gpu_pack_like(hc, geom_of(cfg), [dict(cu=case["cu"], bp=case["bp"], keys=case["keys"],
                                                values=case["values"], radius=r, codes8=c8, codes4=c4,
                                                scores=case["scores"])])
    _compare_caches(dc, hc, "T=32768")


# ---- whole path and the dense baseline -------------------------------------

@pytest.mark.parametrize("number", [1, 2])
def test_pipeline_encode_pack_decode(number):
    """GPU encode -> GPU pack -> GPU decode against oracle encode -> pack -> decode."""
    cfg = synth.WORKLOADS[number]
    case = make_case(cfg)
    flush(f"[pipeline] workload {number}")
    geom = geom_of(cfg)
    hc, _ = oracle_cache(case, maxp=1760 if number == 2 else None)
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, nthreads=8)
    d = _dev_case(case)
    r, c8, c4 = gpu_encode(geom, d["keys"], d["cb8"], d["cb4"])
    dc = ada.Cache(geom, hc.S, hc.maxp, len(hc.arena))
    ada.rdr_pack(geom, dc, case["cu"], case["bp"], d["keys"], d["values"], r, c8, c4, d["scores"])
    out, lse, _ = decode_outputs(geom, dc, d["q"], with_logits=False)
    ada.decode(geom, dc, d["cb8"], d["cb4"], d["q"], cfg.sigma, out, lse)
    torch.cuda.synchronize()
    assert int(dc.cursor[0]) == int(hc.cursor[0])
    err = np.abs(out.cpu().double().numpy() - ref["out"]).max()
    flush(f"[pipeline] workload {number}: out max-abs {err:.2e}")
    assert err <= OUT_TOL


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 32, 8), (64, 4, 4)])
def test_dense_pack_and_decode(D, Hq, Hkv):
    cfg = small_workload(D=D, Hq=Hq, Hkv=Hkv, S=3, T=500, seed=80 + D)
    case = make_case(cfg, lens=[500, 1, 77])
    flush(f"[dense] D={D} Hq={Hq} Hkv={Hkv}")
    geom = geom_of(cfg)
    hc = oracle.HostCache(D, Hkv, 3, 40, 8 << 20, slot_tokens=False)
    n = sum((int(x) + 15) // 16 for x in case["lens"]) * Hkv
    perm = np.random.default_rng(1).permutation(n).astype(np.uint32)
    assert oracle.dense_pack(hc, case["cu"], case["keys"], case["values"], place_perm=perm) == 0
    dc = ada.Cache(geom, 3, 40, 8 << 20)
    d = _dev_case(case)
    ada.dense_pack(geom, dc, case["cu"], d["keys"], d["values"], place_perm=perm)
    torch.cuda.synchronize()
    used = int(hc.cursor[0]) * 128
    assert int(dc.cursor[0]) == int(hc.cursor[0])
    assert np.array_equal(dc.arena[:used].cpu().numpy(), hc.arena[:used])
    ref = oracle.decode(hc, None, None, case["q"], cfg.sigma, logits=True)
    out, lse, lg = decode_outputs(geom, dc, d["q"])
    ada.dense_decode(geom, dc, d["q"], cfg.sigma, out, lse, lg)
    torch.cuda.synchronize()
    ok, worst = logit_tol_ok(lg.cpu().double().numpy(), ref["logits"])
    assert ok, worst
    err = np.abs(out.cpu().double().numpy() - ref["out"]).max()
    flush(f"[dense] out max-abs {err:.2e}")
    assert err <= OUT_TOL


def _sym_tie_codebook(q_head, seed):
    """Codewords A and B of group 0 at the same mathematical distance from the
    query direction u (u_0 = u_1, B is A with coordinates 0 and 1 swapped),
    such that the oracle's arithmetic (each square rounded, then added) ties
    them while a fused multiply-add chain puts B strictly nearer.  Returns
    (A, B) as float32 arrays; the oracle keeps the lower index on the tie."""
    from fractions import Fraction
    x = [float(v) for v in q_head]
    ss = 0.0
    for v in x:
        ss = ss + v * v
    qn = ss ** 0.5
    u = [v / qn for v in x[:8]]
    assert u[0] == u[1]

    def unfused(w):
        d = 0.0
        for j in range(8):
            df = u[j] - float(w[j])
            d = d + df * df
        return d

    def fused(w):
        d = 0.0
        for j in range(8):
            df = Fraction(u[j] - float(w[j]))
            d = float(Fraction(d) + df * df)
        return d

    rng = np.random.default_rng(seed)
    for _ in range(20000):
        a = (np.array(u) + rng.uniform(-0.2, 0.2, 8) * np.array([1, 1, .01, .01, .01, .01, .01, .01]))
        a = a.astype(np.float32)
        b = a.copy()
        b[0], b[1] = a[1], a[0]
        if unfused(a) == unfused(b) and fused(b) < fused(a) and abs(float(a[0]) - float(a[1])) > 0.05:
            return a, b
    raise AssertionError("no near tie found")


def test_decode_sym_query_code_tie_follows_the_oracles_rounding():
    """The symmetric variant's query code is decided in double with each
    square rounded before it is added, as the oracle does.  Two codewords
    that tie under that arithmetic (the lower index wins) but not under a
    fused multiply-add chain must still give the oracle's choice."""
    cfg = small_workload(D=128, Hq=4, Hkv=1, S=1, T=64, seed=8)
    case = make_case(cfg, lens=[64], mixes=[(0, 10000, 10000)])
    q = case["q"].clone()
    q[0, 0, 1] = q[0, 0, 0]
    case["q"] = q
    a, b = _sym_tie_codebook(q[0, 0].double().tolist(), seed=3)
    cb8 = case["cb8"].clone()
    far = -torch.from_numpy(a.astype(np.float32)) - 1.0
    cb8[0, 0, :] = far
    ia, ib = 3, 200
    cb8[0, 0, ia] = torch.from_numpy(a)
    cb8[0, 0, ib] = torch.from_numpy(b)
    case["cb8"] = cb8
    hc, _ = oracle_cache(case)
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True, sym=True)
    # the other choice (B at the lower index) changes the logits far beyond
    # the bar, so a wrong query code cannot pass
    swapped = cb8.clone()
    swapped[0, 0, ia], swapped[0, 0, ib] = cb8[0, 0, ib], cb8[0, 0, ia]
    hc2, _ = oracle_cache(dict(case, cb8=swapped))
    alt = oracle.decode(hc2, swapped, case["cb4"], case["q"], cfg.sigma, logits=True, sym=True)
    m = ~np.isnan(ref["logits"][0, 0])
    assert np.abs(alt["logits"][0, 0][m] - ref["logits"][0, 0][m]).max() > 1e-2 * np.abs(ref["logits"][0, 0][m]).max()
    geom = geom_of(cfg)
    dc = upload_cache(hc, geom)
    d = _dev_case(case)
    flush("[decode_sym] query-code tie")
    out, lse, lg = decode_outputs(geom, dc, d["q"])
    ada.decode_sym(geom, dc, d["cb8"], d["cb4"], d["q"], cfg.sigma, out, lse, lg, num_splits=1)
    torch.cuda.synchronize()
    ok, worst = logit_tol_ok(lg.cpu().double().numpy(), ref["logits"])
    assert ok, f"logits off by {worst:.3g} (relative)"


def test_decode_sym_query_norm_wide_range_and_exact_tree():
    """The symmetric variant's |q| is the squares summed in order in double.
    The kernel sums them in a tree when that sum is provably exact, else in
    order: one head whose squares span far more than 53 bits takes the
    ordered sum, the others the tree; both must give the oracle's codes."""
    cfg = small_workload(D=128, Hq=4, Hkv=1, S=1, T=96, seed=12)
    case = make_case(cfg, lens=[96], mixes=[(1000, 6000, 9000)])
    q = case["q"].float().clone()
    q[0, 0, 0::2] *= 2.0 ** 50
    q[0, 0, 1::2] *= 2.0 ** -50
    q[0, 1] *= 2.0 ** -100
    case["q"] = q.to(torch.bfloat16)
    hc, _ = oracle_cache(case)
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True, sym=True)
    geom = geom_of(cfg)
    dc = upload_cache(hc, geom)
    d = _dev_case(case)
    flush("[decode_sym] wide-range query norms")
    out, lse, lg = decode_outputs(geom, dc, d["q"])
    ada.decode_sym(geom, dc, d["cb8"], d["cb4"], d["q"], cfg.sigma, out, lse, lg, num_splits=1)
    torch.cuda.synchronize()
    ok, worst = logit_tol_ok(lg.cpu().double().numpy(), ref["logits"])
    assert ok, f"logits off by {worst:.3g} (relative)"


def test_decode_sym_llama_shape_t32k_full():
    """The symmetric variant at full size (one T=32768 sequence, 32/8 heads,
    D=128) in the bench's launch configuration (default splits) and with 7
    splits: every logit, output and lse against the oracle's."""
    cfg = synth.WORKLOADS[2]
    case = make_case(cfg)
    hc, _ = oracle_cache(case, maxp=1760)
    ref = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True, nthreads=16, sym=True)
    geom = geom_of(cfg)
    dc = upload_cache(hc, geom)
    d = _dev_case(case)
    for sp in (0, 7):
        flush(f"[decode_sym] Llama-3-8B shape T=32768 splits={sp}")
        out, lse, lg = decode_outputs(geom, dc, d["q"])
        ada.decode_sym(geom, dc, d["cb8"], d["cb4"], d["q"], cfg.sigma, out, lse, lg, num_splits=sp)
        torch.cuda.synchronize()
        ok, worst = logit_tol_ok(lg.cpu().double().numpy(), ref["logits"])
        assert ok, f"logits off by {worst:.3g} (relative)"
        err = np.abs(out.cpu().double().numpy() - ref["out"]).max()
        assert err <= OUT_TOL, f"out max-abs {err:.3g}"
        l = lse.cpu().double().numpy()
        assert (np.abs(l - ref["lse"]) <= 1e-3 * np.maximum(np.abs(ref["lse"]), 1.0)).all()


def test_dense_llama_shape_t32k_full():
    """The dense bf16 comparison path at full size (one T=32768 sequence,
    8 kv-heads, D=128): pages bit-exact, every logit and output against the
    oracle's dense decode."""
    cfg = synth.WORKLOADS[2]
    case = make_case(cfg)
    D, H, T = cfg.head_dim, cfg.num_kv_heads, int(case["lens"][0])
    maxp = T // 16 + 4
    nbytes = T * H * 4 * D + H * 8192
    hc = oracle.HostCache(D, H, 1, maxp, nbytes, slot_tokens=False)
    assert oracle.dense_pack(hc, case["cu"], case["keys"], case["values"]) == 0
    geom = geom_of(cfg)
    dc = ada.Cache(geom, 1, maxp, nbytes)
    d = _dev_case(case)
    flush("[dense] Llama-3-8B shape T=32768")
    ada.dense_pack(geom, dc, case["cu"], d["keys"], d["values"])
    torch.cuda.synchronize()
    used = int(hc.cursor[0]) * 128
    assert int(dc.cursor[0]) == int(hc.cursor[0])
    assert np.array_equal(dc.arena[:used].cpu().numpy(), hc.arena[:used])
    ref = oracle.decode(hc, None, None, case["q"], cfg.sigma, logits=True, nthreads=16)
    out, lse, lg = decode_outputs(geom, dc, d["q"])
    ada.dense_decode(geom, dc, d["q"], cfg.sigma, out, lse, lg)
    torch.cuda.synchronize()
    ok, worst = logit_tol_ok(lg.cpu().double().numpy(), ref["logits"])
    assert ok, f"logits off by {worst:.3g} (relative)"
    err = np.abs(out.cpu().double().numpy() - ref["out"]).max()
    flush(f"[dense] full size out max-abs {err:.2e}")
    assert err <= OUT_TOL
