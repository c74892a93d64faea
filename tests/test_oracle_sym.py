"""Pins for the oracle's symmetric (query-code) decode variant (CPU only).

The query's direction takes per-group codes like a key, and coded logits
become sigma |q| r~ sum_g C_g[cq_g] . C_g[ck_g].  Pinned by: the query codes
against brute force over every codeword, exactness when the query's
direction slices are codewords (the variant then equals the asymmetric
decode), the table form against the rebuilt-vectors form, scale behaviour,
and fp16-tier logits that do not change."""
import numpy as np
import pytest
import torch

import oracle
from helpers import make_case, oracle_cache, small_workload


def _q_f64(q):
    return q.float().double().numpy()


def test_query_codes_match_brute_force():
    cfg = small_workload(D=128, Hq=8, Hkv=2, S=3, T=16, seed=21)
    case = make_case(cfg)
    qc8, qc4, qn = oracle.query_codes(case["q"], case["cb8"], case["cb4"])
    q = _q_f64(case["q"])
    cb8, cb4 = case["cb8"].double().numpy(), case["cb4"].double().numpy()
    S, Hq, D = q.shape
    for s in range(S):
        for h in range(Hq):
            kv = h // (Hq // 2)
            n = np.sqrt(np.sum(q[s, h] ** 2))
            assert abs(qn[s, h] - n) <= 1e-12 * n
            u = q[s, h] / n
            for g in range(D // 8):
                d8 = ((u[8 * g: 8 * g + 8] - cb8[kv, g]) ** 2).sum(1)
                d4 = ((u[8 * g: 8 * g + 8] - cb4[kv, g]) ** 2).sum(1)
                assert d8[qc8[s, h, g]] <= d8.min() + 1e-12 and d4[qc4[s, h, g]] <= d4.min() + 1e-12


def _codebooks_holding_query(case, kv_of):
    """Codebooks in which codeword 7 (8-bit) and 3 (4-bit) of every group are
    the fp32-rounded direction slices of that kv-head's (single) query."""
    cb8 = case["cb8"].clone()
    cb4 = case["cb4"].clone()
    q = _q_f64(case["q"])
    for h, kv in enumerate(kv_of):
        u = q[0, h] / np.sqrt(np.sum(q[0, h] ** 2))
        for g in range(q.shape[2] // 8):
            cb8[kv, g, 7] = torch.from_numpy(u[8 * g: 8 * g + 8]).float()
            cb4[kv, g, 3] = torch.from_numpy(u[8 * g: 8 * g + 8]).float()
    return cb8, cb4


@pytest.mark.parametrize("D", [64, 128])
def test_sym_equals_asym_when_the_query_is_a_codeword(D):
    cfg = small_workload(D=D, Hq=2, Hkv=2, S=1, T=300, seed=22 + D)
    case = make_case(cfg)
    cb8, cb4 = _codebooks_holding_query(case, [0, 1])
    case["cb8"], case["cb4"] = cb8, cb4
    qc8, qc4, _ = oracle.query_codes(case["q"], cb8, cb4)
    assert (qc8 == 7).all() and (qc4 == 3).all()
    hc, _ = oracle_cache(case)
    a = oracle.decode(hc, cb8, cb4, case["q"], cfg.sigma, logits=True)
    b = oracle.decode(hc, cb8, cb4, case["q"], cfg.sigma, logits=True, sym=True)
    m = ~np.isnan(a["logits"])
    # the codewords hold u_q rounded to fp32 (relative 2^-24), so logits
    # agree to about sigma r~ |q| |C| 2^-24 < 1e-6 here
    assert np.allclose(b["logits"][m], a["logits"][m], rtol=1e-6, atol=2e-6)
    assert np.abs(b["out"] - a["out"]).max() < 1e-6


def test_sym_table_form_equals_rebuilt_vectors_and_fp16_tier_unchanged():
    cfg = small_workload(D=128, Hq=4, Hkv=2, S=2, T=200, seed=23)
    case = make_case(cfg, lens=[200, 77])
    hc, _ = oracle_cache(case)
    a = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True)
    b = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True, sym=True)
    m = ~np.isnan(b["logits"])
    assert np.allclose(b["logits"][m], b["logits_explicit"][m], rtol=1e-12, atol=1e-12)
    # slots of fp16 pages keep sigma q . k; coded slots move
    tier = np.full(b["logits"].shape[2], -1)
    same = np.isclose(a["logits"], b["logits"], rtol=0, atol=0) & m
    for row in range(hc.S * hc.Hkv):
        s, kv = divmod(row, hc.Hkv)
        for p in range(hc.num_pages[row]):
            t = hc.page_meta[row, p] & 3
            for h in range(kv * 2, kv * 2 + 2):
                sl = slice(16 * p, 16 * p + 16)
                mm = m[s, h, sl]
                if t == 0:
                    assert same[s, h, sl][mm].all()
                else:
                    assert not same[s, h, sl][mm].all()


def test_sym_logits_scale_with_the_query_and_codes_do_not():
    cfg = small_workload(D=64, Hq=4, Hkv=2, S=1, T=150, seed=24)
    case = make_case(cfg)
    hc, _ = oracle_cache(case)
    q2 = (case["q"].float() * 4).to(torch.bfloat16)  # exact: a power of two
    c1 = oracle.query_codes(case["q"], case["cb8"], case["cb4"])
    c2 = oracle.query_codes(q2, case["cb8"], case["cb4"])
    assert np.array_equal(c1[0], c2[0]) and np.array_equal(c1[1], c2[1])
    a = oracle.decode(hc, case["cb8"], case["cb4"], case["q"], cfg.sigma, logits=True, sym=True)
    b = oracle.decode(hc, case["cb8"], case["cb4"], q2, cfg.sigma, logits=True, sym=True)
    m = ~np.isnan(a["logits"])
    assert np.allclose(b["logits"][m], 4 * a["logits"][m], rtol=1e-12, atol=1e-12)
