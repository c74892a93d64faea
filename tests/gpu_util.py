"""Helpers for GPU parity tests: move oracle-built caches to the device and run
the library's encode/pack through the binding."""
from __future__ import annotations

import numpy as np
import torch

import compressed_kv_attention_amd as ada


def geom_of(cfg) -> ada.Geom:
    return ada.Geom(cfg.head_dim, cfg.num_q_heads, cfg.num_kv_heads)


def u16(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)


def to_dev(x) -> torch.Tensor:
    """numpy array or CPU tensor -> contiguous device tensor (uint16 arrays
    come back as int16 bit patterns)."""
    if isinstance(x, np.ndarray):
        x = np.ascontiguousarray(x)
        if x.dtype == np.uint16:
            x = x.view(np.int16)
        x = torch.from_numpy(x)
    return x.contiguous().cuda()


def upload_cache(hc, geom: ada.Geom, slot_tokens=False) -> ada.Cache:
    """An ada.Cache holding exactly the bytes and tables of an oracle cache."""
    c = ada.Cache(geom, hc.S, hc.maxp, len(hc.arena), slot_tokens=slot_tokens)
    c.arena.copy_(torch.from_numpy(hc.arena))
    c.page_table.copy_(torch.from_numpy(hc.page_table.view(np.int32)))
    c.page_meta.copy_(torch.from_numpy(hc.page_meta))
    c.num_pages[: len(hc.num_pages)].copy_(torch.from_numpy(hc.num_pages))
    c.tier_tokens[: len(hc.tier_tokens)].copy_(torch.from_numpy(hc.tier_tokens))
    c.cursor[:] = hc.cursor
    c.num_pages_host[: len(hc.num_pages)] = hc.num_pages
    return c


def gpu_encode(geom, keys_dev, cb8_dev, cb4_dev):
    n = keys_dev.shape[0]
    H, D = geom.num_kv_heads, geom.head_dim
    r = torch.empty((n, H), dtype=torch.float16, device=keys_dev.device)
    c8 = torch.empty((n, H, D // 8), dtype=torch.uint8, device=keys_dev.device)
    c4 = torch.empty((n, H, D // 16), dtype=torch.uint8, device=keys_dev.device)
    ada.encode(geom, keys_dev, cb8_dev, cb4_dev, r, c8, c4)
    return r, c8, c4


def decode_outputs(geom, cache, q_dev, with_logits=True, lse=True):
    S, Hq, D = cache.num_seqs, geom.num_q_heads, geom.head_dim
    out = torch.full((S, Hq, D), float("nan"), device="cuda")
    ls = torch.full((S, Hq), float("nan"), device="cuda") if lse else None
    lg = torch.full((S, Hq, cache.maxp * 16), float("nan"), device="cuda") if with_logits else None
    return out, ls, lg


def logit_tol_ok(got, ref):
    """|d| <= 1e-3 * max(|ref|, 1e-2) on every retained slot."""
    m = ~np.isnan(ref)
    g, r = got[m], ref[m]
    if np.isnan(g).any():
        return False, float("nan")
    err = np.abs(g - r) / np.maximum(np.abs(r), 1e-2)
    return bool((err <= 1e-3).all()), float(err.max(initial=0.0))


def flush(msg: str):
    print(msg, flush=True)
