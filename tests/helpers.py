"""Shared test helpers: small seeded cases and oracle-built caches."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synth
from synth.configs import Workload

_SMALL_ID = [200]


def small_workload(D=64, Hq=4, Hkv=2, S=1, T=128, mix=(2500, 7500, 10000), seed=0,
                   outliers=True, samples=1024, iters=4) -> Workload:
    return Workload(300 + seed, f"small-{seed}", S, 1, Hq, Hkv, D, T, tier_cum_bp=tuple(mix),
                    key_outliers=outliers, codebook_samples=samples, lloyd_iters=iters)


def make_case(cfg: Workload, layer=0, lens=None, mixes=None, device="cpu"):
    """Inputs of one layer: dict of torch tensors (CPU unless device given)."""
    if lens is None:
        lens = synth.seq_lens(cfg)
    lens = np.asarray(lens, dtype=np.int64)
    cu = synth.cu_tokens(lens)
    N = int(cu[-1])
    bp = synth.tier_mix(cfg) if mixes is None else np.asarray(mixes, dtype=np.int32)
    cb8, cb4 = synth.codebooks(cfg, layer)
    return dict(
        cfg=cfg, lens=lens, cu=cu, bp=bp, N=N,
        keys=synth.keys(cfg, layer, N, device),
        values=synth.values(cfg, layer, N, device),
        scores=synth.scores(cfg, layer, N),
        q=synth.queries(cfg, layer, device),
        cb8=cb8, cb4=cb4,
    )


def oracle_cache(case, maxp=None, arena_bytes=None, protect=None, place_perm=None, slot_tokens=True):
    """Encode + pack a case with the oracle; returns (HostCache, encode outputs)."""
    cfg = case["cfg"]
    D, H = cfg.head_dim, cfg.num_kv_heads
    r, c8, c4 = oracle.encode(case["keys"], case["cb8"], case["cb4"])
    S = len(case["lens"])
    if maxp is None:
        maxp = int(max(case["lens"]) // 16 + 4)
    if arena_bytes is None:
        arena_bytes = int(sum(case["lens"]) * H * 512 + S * H * 3 * 8192 + 4096)
    cache = oracle.HostCache(D, H, S, maxp, arena_bytes, slot_tokens=slot_tokens)
    rc = oracle.pack(cache, case["cu"], case["bp"], case["keys"], case["values"], r, c8, c4,
                     case["scores"], protect=protect, place_perm=place_perm)
    assert rc == 0, rc
    return cache, (r, c8, c4)


def bf16_bits_to_f64(x) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    return t.double().numpy()


def f16_bits_to_f64(x) -> np.ndarray:
    return np.ascontiguousarray(x).view(np.float16).astype(np.float64)
