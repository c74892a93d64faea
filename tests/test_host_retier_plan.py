"""The library's host-side re-tiering policy (ada_retier_plan, no device
work) against the oracle's on random page tables (CPU only)."""
import numpy as np
import pytest

import compressed_kv_attention_amd as ada
import oracle


@pytest.mark.parametrize("seed", range(6))
def test_retier_plan_matches_oracle(seed):
    rng = np.random.default_rng(seed)
    D = 128 if seed % 2 else 64
    S, H, maxp = 3, 2, 24
    hc = oracle.HostCache(D, H, S, maxp, 1 << 12, slot_tokens=False)
    hc.num_pages[:] = rng.integers(0, maxp + 1, S * H)
    tiers = rng.integers(0, 3, (S * H, maxp))
    fill = np.where(rng.random((S * H, maxp)) < 0.7, 15, rng.integers(0, 15, (S * H, maxp)))
    hc.page_meta[:] = (tiers | (fill << 2)).astype(np.uint8)
    used = np.array([sum(oracle.page_bytes(D, int(hc.page_meta[r, p]) & 3)
                         for r in range(s * H, s * H + H) for p in range(hc.num_pages[r])) for s in range(S)])
    budgets = (used * rng.uniform(0.0, 1.2, S)).astype(np.int64)
    g = ada.Geom(D, 2 * H, H)
    for demote_to in (1, 2):
        for cap in (1 << 12, 5):
            a = ada.retier_plan(g, budgets, hc.num_pages, hc.page_meta, demote_to=demote_to, cap=cap)
            b = oracle.retier_plan(hc, budgets, demote_to=demote_to, cap=cap)
            for x, y in zip(a, b):
                assert np.array_equal(x, y)
