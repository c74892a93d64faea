"""Pins for the oracle's decode step (CPU only).

I1  an all-fp16, no-drop cache is textbook softmax attention (checked against
    torch's scaled_dot_product_attention in float64);
I2  each code-table logit equals r~ * (q . c^) with the coded key rebuilt;
I3  dropped tokens contribute nothing (perturbing them changes no bit);
I4  softmax weights sum to one through lse;
I5  one retained token gives its value back; q = 0 gives the mean value;
I6  a codebook holding the exact directions gives dense attention with the
    fp16 radius;
I8  an MHA run equals a GQA run with replicated KV heads;
plus the empty row and the dense bf16 comparison cache."""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from helpers import bf16_bits_to_f64, f16_bits_to_f64, make_case, oracle_cache, small_workload
from pagefmt import read_page


def _sdpa(q, K, V, sigma):
    """torch reference in float64: q [D], K/V [n][D]."""
    out = F.scaled_dot_product_attention(
        torch.from_numpy(q)[None, None, None], torch.from_numpy(K)[None, None],
        torch.from_numpy(V)[None, None], scale=sigma)
    logits = sigma * (K @ q)
    m = logits.max()
    return out[0, 0, 0].numpy(), m + np.log(np.exp(logits - m).sum())


def test_dense_attention_matches_torch_sdpa():
    rng = np.random.default_rng(0)
    for n in (1, 5, 300):
        q, K, V = rng.standard_normal(64), rng.standard_normal((n, 64)), rng.standard_normal((n, 64))
        out, lse = oracle.dense_attention(q, K, V, 0.125)
        ref, rlse = _sdpa(q, K, V, 0.125)
        assert np.allclose(out, ref, rtol=0, atol=1e-12)
        assert abs(lse - rlse) < 1e-12
    out, lse = oracle.dense_attention(np.ones(8), np.zeros((0, 8)), np.zeros((0, 8)), 1.0)
    assert not out.any() and lse == -np.inf


@pytest.mark.parametrize("D,Hq,Hkv", [(64, 4, 4), (128, 8, 2)])
def test_I1_all_fp16_no_drop_is_softmax_attention(D, Hq, Hkv):
    cfg = small_workload(D=D, Hq=Hq, Hkv=Hkv, S=2, T=70, mix=(10000, 10000, 10000), seed=20)
    case = make_case(cfg, lens=[70, 33])
    cache, _ = oracle_cache(case)
    res = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    K = case["keys"].double().numpy()
    V = case["values"].double().numpy()
    q = case["q"].double().numpy()
    cu = case["cu"]
    for s in range(2):
        for hq in range(Hq):
            h = hq // (Hq // Hkv)
            ref, rlse = _sdpa(q[s, hq], K[cu[s]:cu[s + 1], h], V[cu[s]:cu[s + 1], h], cfg.sigma)
            assert np.allclose(res["out"][s, hq], ref, rtol=0, atol=1e-12)
            assert abs(res["lse"][s, hq] - rlse) < 1e-12


def test_I2_code_table_logits_equal_rebuilt_key_logits_and_I4():
    cfg = small_workload(D=128, Hq=8, Hkv=2, S=2, T=90, mix=(2000, 6000, 9000), seed=21)
    case = make_case(cfg)
    cache, _ = oracle_cache(case)
    res = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True)
    lg, lx = res["logits"], res["logits_explicit"]
    m = ~np.isnan(lg)
    assert np.array_equal(m, ~np.isnan(lx))
    assert np.allclose(lg[m], lx[m], rtol=1e-12, atol=1e-12)
    # I4: sum_t exp(l_t - lse) = 1
    for s in range(2):
        for hq in range(8):
            row = lg[s, hq][~np.isnan(lg[s, hq])]
            assert abs(np.exp(row - res["lse"][s, hq]).sum() - 1.0) < 1e-12
    # every retained slot has a logit: 90 * 0.9 = 81 per row
    assert (m.sum(-1) == 81).all()


def test_I2_logit_of_a_coded_slot_by_hand():
    """One 8-bit slot: rebuild c^ from the codes read out of the page and
    compare the oracle's logit with sigma * r~ * q . c^ computed here."""
    cfg = small_workload(D=64, Hq=1, Hkv=1, S=1, T=16, mix=(0, 10000, 10000), seed=22)
    case = make_case(cfg)
    cache, _ = oracle_cache(case)
    res = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True)
    pg = read_page(cache.page(0, 0), 64, 1)
    q = case["q"].double().numpy()[0, 0]
    cb = case["cb8"].double().numpy()[0]
    for t in range(16):
        chat = np.concatenate([cb[g, pg["codes"][t, g]] for g in range(8)])
        r = f16_bits_to_f64(pg["radius"][t:t + 1])[0]
        assert abs(res["logits"][0, 0, t] - cfg.sigma * r * (q @ chat)) < 1e-12


def test_I3_dropped_tokens_contribute_nothing():
    cfg = small_workload(D=64, Hq=4, Hkv=2, S=1, T=120, mix=(2000, 5000, 7000), seed=23)
    case = make_case(cfg)
    cache, enc = oracle_cache(case)
    base = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    # find dropped (token, head) pairs and scramble their K, V and codes
    kept = set()
    for row in range(2):
        for p in range(cache.num_pages[row]):
            for t in cache.slot_token[row, p]:
                if t >= 0:
                    kept.add((int(t), row))
    dropped = [(t, h) for t in range(120) for h in range(2) if (t, h) not in kept]
    assert len(dropped) == 2 * (120 - 84)
    keys, vals = case["keys"].clone(), case["values"].clone()
    for t, h in dropped:
        keys[t, h] = -keys[t, h] * 7
        vals[t, h] = 1000.0
    case2 = dict(case, keys=keys, values=vals)
    r, c8, c4 = oracle.encode(keys, case["cb8"], case["cb4"])
    cache2 = oracle.HostCache(64, 2, 1, cache.maxp, len(cache.arena))
    assert oracle.pack(cache2, case["cu"], case["bp"], keys, vals, r, c8, c4, case["scores"]) == 0
    got = oracle.decode(cache2, case2["cb8"], case2["cb4"], case["q"], cfg.sigma)
    assert np.array_equal(got["out"], base["out"]) and np.array_equal(got["lse"], base["lse"])


@pytest.mark.parametrize("tier_bp", [(10000, 10000, 10000), (0, 10000, 10000), (0, 0, 10000)])
def test_I5_single_token_returns_its_value(tier_bp):
    cfg = small_workload(D=128, Hq=4, Hkv=1, S=1, T=1, mix=tier_bp, seed=24)
    case = make_case(cfg)
    cache, _ = oracle_cache(case)
    res = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    tier = int(cache.page_meta[0, 0]) & 3
    pg = read_page(cache.page(0, 0), 128, tier)
    if tier == 2:
        vhat = pg["Vq"][0].astype(np.float64) * f16_bits_to_f64(pg["vscale"][:1])[0]
    else:
        vhat = bf16_bits_to_f64(pg["V"][0])
    for hq in range(4):
        assert np.allclose(res["out"][0, hq], vhat, rtol=0, atol=1e-15)


def test_I5_zero_query_gives_mean_value():
    cfg = small_workload(D=64, Hq=2, Hkv=1, S=1, T=50, mix=(2000, 6000, 8000), seed=25)
    case = make_case(cfg)
    cache, _ = oracle_cache(case)
    q0 = torch.zeros_like(case["q"])
    res = oracle.decode(cache, case["cb8"], case["cb4"], q0, cfg.sigma)
    vs = []
    for p in range(cache.num_pages[0]):
        meta = int(cache.page_meta[0, p])
        tier, nv = meta & 3, ((meta >> 2) & 15) + 1
        pg = read_page(cache.page(0, p), 64, tier)
        for t in range(nv):
            if tier == 2:
                vs.append(pg["Vq"][t].astype(np.float64) * f16_bits_to_f64(pg["vscale"][t:t + 1])[0])
            else:
                vs.append(bf16_bits_to_f64(pg["V"][t]))
    assert len(vs) == 40
    assert np.allclose(res["out"][0, 0], np.mean(vs, 0), rtol=0, atol=1e-13)
    assert abs(res["lse"][0, 0] - np.log(40)) < 1e-13


def test_I6_exact_direction_codebook_gives_dense_attention_with_fp16_radius():
    cfg = small_workload(D=64, Hq=2, Hkv=1, S=1, T=200, mix=(0, 10000, 10000), seed=26)
    case = make_case(cfg)
    k = case["keys"].double().numpy()[:, 0]  # [T][D]
    r = np.sqrt((k * k).sum(-1))
    u = k / r[:, None]
    cb8 = np.zeros((1, 8, 256, 8), np.float32)
    for t in range(200):
        cb8[0, :, t, :] = u[t].reshape(8, 8)
    case["cb8"] = torch.from_numpy(cb8)
    cache, (rt, c8, _) = oracle_cache(case)
    assert np.array_equal(c8[:, 0], np.tile(np.arange(200)[:, None], (1, 8)))
    res = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    rtil = f16_bits_to_f64(rt[:, 0])
    Kq = rtil[:, None] * cb8[0].transpose(1, 0, 2).reshape(256, 64)[:200].astype(np.float64)
    V = case["values"].double().numpy()[:, 0]
    q = case["q"].double().numpy()[0]
    for hq in range(2):
        ref, rlse = _sdpa(q[hq], Kq, V, cfg.sigma)
        assert np.allclose(res["out"][0, hq], ref, rtol=0, atol=1e-12)
        # against the unquantized keys the only differences are fp16 radius
        # and fp32 codebook rounding
        ref2, _ = _sdpa(q[hq], k, V, cfg.sigma)
        assert np.allclose(res["out"][0, hq], ref2, rtol=0, atol=5e-3)


def test_I8_mha_equals_gqa_with_replicated_kv_heads():
    cfg = small_workload(D=64, Hq=4, Hkv=1, S=1, T=60, mix=(2500, 6000, 9000), seed=27)
    case = make_case(cfg)
    gqa_cache, _ = oracle_cache(case)
    gqa = oracle.decode(gqa_cache, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    rep = dict(case)
    for k in ("keys", "values", "scores"):
        rep[k] = case[k].repeat_interleave(4, dim=1)
    rep["cb8"] = case["cb8"].repeat(4, 1, 1, 1)
    rep["cb4"] = case["cb4"].repeat(4, 1, 1, 1)
    rep["cfg"] = small_workload(D=64, Hq=4, Hkv=4, S=1, T=60, mix=(2500, 6000, 9000), seed=27)
    mha_cache, _ = oracle_cache(rep)
    mha = oracle.decode(mha_cache, rep["cb8"], rep["cb4"], case["q"], cfg.sigma)
    assert np.array_equal(gqa["out"], mha["out"]) and np.array_equal(gqa["lse"], mha["lse"])


def test_empty_row_gives_zero_output_and_minus_inf_lse():
    cfg = small_workload(D=64, Hq=2, Hkv=1, S=3, T=40, mix=(2500, 6000, 9000), seed=28)
    case = make_case(cfg, lens=[40, 0, 1], mixes=[(2500, 6000, 9000), (2500, 6000, 9000), (0, 0, 0)])
    cache, _ = oracle_cache(case)
    res = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    for s in (1, 2):  # no tokens / only a dropped token
        assert not res["out"][s].any()
        assert (res["lse"][s] == -np.inf).all()
    assert np.isfinite(res["lse"][0]).all()


def test_dense_bf16_cache_is_softmax_attention_over_bf16_keys():
    cfg = small_workload(D=128, Hq=4, Hkv=2, S=1, T=45, seed=29)
    case = make_case(cfg)
    cache = oracle.HostCache(128, 2, 1, 8, 1 << 20, slot_tokens=False)
    assert oracle.dense_pack(cache, case["cu"], case["keys"], case["values"]) == 0
    assert (cache.page_meta[:, :3] & 3 == 3).all()
    res = oracle.decode(cache, None, None, case["q"], cfg.sigma)
    Kb = case["keys"].to(torch.bfloat16).double().numpy()
    V = case["values"].double().numpy()
    q = case["q"].double().numpy()
    for hq in range(4):
        ref, rlse = _sdpa(q[0, hq], Kb[:, hq // 2], V[:, hq // 2], cfg.sigma)
        assert np.allclose(res["out"][0, hq], ref, rtol=0, atol=1e-12)
        assert abs(res["lse"][0, hq] - rlse) < 1e-12


def test_units_range_and_threads_do_not_change_results():
    cfg = small_workload(D=64, Hq=4, Hkv=2, S=2, T=64, seed=30)
    case = make_case(cfg)
    cache, _ = oracle_cache(case)
    a = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma)
    b = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma, nthreads=3)
    c = oracle.decode(cache, case["cb8"], case["cb4"], case["q"], cfg.sigma, units=(2, 5))
    assert np.array_equal(a["out"], b["out"])
    assert np.array_equal(a["out"].reshape(8, -1)[2:5], c["out"].reshape(8, -1)[2:5])
