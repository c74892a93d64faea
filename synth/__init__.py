"""Seeded synthetic inputs for the ADA decode path.

This module feeds both sides of every parity check (the CPU oracle and the HIP
library) and the benchmark.  It holds none of the method's arithmetic: it
draws keys, values, queries and utility scores, and fits the per-head
codebooks that the method takes as given inputs (the way a model's weights are
given).  Nothing here encodes, ranks, packs or attends.

Distributions (the pages give none; these follow the workload table):
  * per (layer, kv-head, channel) scale s = exp(0.5 z), z ~ N(0, 1);
  * where a workload has key outliers, round(1% of D) (at least one) channels
    per (layer, kv-head), drawn without replacement, get 8x their scale;
  * keys  = N(0, 1) * s, rounded to fp16;
  * values = N(0, 1) (times a second scale draw where the workload says so),
    rounded to bf16;
  * queries = N(0, 1), rounded to bf16;
  * utility scores: Zipf(a = 1.1) integer draws per (token, kv-head), clipped
    to [1, 2^24], as float32 (higher = more useful);
  * codebooks: per (layer, kv-head, group of 8 dims) k-means on 4096 sampled
    directions of that head's own key distribution: 10 Lloyd iterations,
    start = the first K samples of a seeded shuffle, an empty cluster keeps
    its centroid, 256 codewords (8-bit tier) and 16 (4-bit tier).

Small workloads are drawn on the CPU with numpy (bit-identical everywhere);
the large ones are drawn on the GPU with torch's seeded generator, and a test
that needs a sample on the CPU copies that slice back.
"""
from __future__ import annotations

import hashlib

import numpy as np
import torch

from .configs import WORKLOADS, Workload, mix_for_budget, stored_fraction  # noqa: F401


def _seed(*parts) -> int:
    h = hashlib.sha256(repr(parts).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _rng(*parts) -> np.random.Generator:
    return np.random.default_rng(_seed(*parts))


def channel_scales(cfg: Workload, layer: int, kind: str) -> np.ndarray:
    """[Hkv][D] float32 channel scales for 'key' or 'value'."""
    rng = _rng(cfg.seed, layer, "scale", kind)
    s = np.exp(0.5 * rng.standard_normal((cfg.num_kv_heads, cfg.head_dim))).astype(np.float32)
    if kind == "key" and cfg.key_outliers:
        n_out = max(1, int(round(0.01 * cfg.head_dim)))
        for h in range(cfg.num_kv_heads):
            ch = rng.choice(cfg.head_dim, size=n_out, replace=False)
            s[h, ch] *= 8.0
    return s


def seq_lens(cfg: Workload) -> np.ndarray:
    if cfg.seq_len is not None:
        return np.full(cfg.num_seqs, cfg.seq_len, dtype=np.int64)
    lo, hi = cfg.len_range
    return _rng(cfg.seed, "lens").integers(lo, hi + 1, size=cfg.num_seqs).astype(np.int64)


def budgets_bp(cfg: Workload) -> np.ndarray:
    """[S] int64 byte budget of each sequence, in basis points of its dense
    bf16 cache: drawn per sequence where the workload gives a range, else the
    workload's fixed budget."""
    if cfg.budget_range_bp is None:
        return np.full(cfg.num_seqs, cfg.budget_bp, dtype=np.int64)
    lo, hi = cfg.budget_range_bp
    return _rng(cfg.seed, "budgets").integers(lo, hi + 1, size=cfg.num_seqs).astype(np.int64)


def budget_bytes(cfg: Workload, lens) -> np.ndarray:
    """[S] int64 byte budget per sequence for the budget solver: the budget's
    share of the dense bf16 cache (K and V, 2 bytes each per dim) of the
    sequence's tokens, rounded down."""
    dense = np.asarray(lens, dtype=np.int64) * cfg.num_kv_heads * 4 * cfg.head_dim
    return dense * budgets_bp(cfg) // 10000


def tier_mix(cfg: Workload) -> np.ndarray:
    """[S][3] int32 cumulative basis points per sequence."""
    if cfg.tier_cum_bp is not None:
        return np.tile(np.array(cfg.tier_cum_bp, dtype=np.int32), (cfg.num_seqs, 1))
    return np.array([mix_for_budget(int(b)) for b in budgets_bp(cfg)], dtype=np.int32)


def cu_tokens(lens) -> np.ndarray:
    out = np.zeros(len(lens) + 1, dtype=np.int32)
    out[1:] = np.cumsum(lens)
    return out


def _to_bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def _normal(shape, seed_parts, device) -> torch.Tensor:
    if str(device) == "cpu":
        a = _rng(*seed_parts).standard_normal(shape, dtype=np.float32)
        return torch.from_numpy(a)
    g = torch.Generator(device=device)
    g.manual_seed(_seed(*seed_parts))
    return torch.randn(shape, generator=g, device=device, dtype=torch.float32)


def keys(cfg: Workload, layer: int, n_tokens: int, device="cpu", stream: str = "k") -> torch.Tensor:
    """[n][Hkv][D] fp16 keys."""
    s = torch.from_numpy(channel_scales(cfg, layer, "key")).to(device)
    z = _normal((n_tokens, cfg.num_kv_heads, cfg.head_dim), (cfg.seed, layer, stream), device)
    return (z * s).to(torch.float16)


def values(cfg: Workload, layer: int, n_tokens: int, device="cpu", stream: str = "v") -> torch.Tensor:
    """[n][Hkv][D] bf16 values."""
    z = _normal((n_tokens, cfg.num_kv_heads, cfg.head_dim), (cfg.seed, layer, stream), device)
    if cfg.value_scaled:
        z = z * torch.from_numpy(channel_scales(cfg, layer, "value")).to(device)
    return _to_bf16(z)


def queries(cfg: Workload, layer: int, device="cpu", step: int = 0) -> torch.Tensor:
    """[S][Hq][D] bf16 queries."""
    z = _normal((cfg.num_seqs, cfg.num_q_heads, cfg.head_dim), (cfg.seed, layer, "q", step), device)
    return _to_bf16(z)


def scores(cfg: Workload, layer: int, n_tokens: int, stream: str = "score") -> torch.Tensor:
    """[n][Hkv] float32 utility scores (drawn on the CPU)."""
    z = _rng(cfg.seed, layer, stream).zipf(1.1, size=(n_tokens, cfg.num_kv_heads))
    return torch.from_numpy(np.minimum(z, 1 << 24).astype(np.float32))


def _lloyd(x: torch.Tensor, k: int, iters: int, perm: torch.Tensor, chunk: int = 16) -> torch.Tensor:
    """Batched k-means on the CPU.  x [B][n][8] float32 -> centroids [B][k][8]."""
    out = []
    for b0 in range(0, x.shape[0], chunk):
        xb = x[b0:b0 + chunk]
        c = xb[:, perm[:k], :].clone()
        x2 = (xb * xb).sum(-1, keepdim=True)
        for _ in range(iters):
            # squared distances in expanded form; argmin takes the lowest index on ties
            d = x2 - 2.0 * (xb @ c.transpose(1, 2)) + (c * c).sum(-1)[:, None, :]
            a = d.argmin(-1)  # [b][n]
            sums = torch.zeros_like(c).scatter_add_(1, a[..., None].expand(-1, -1, 8), xb)
            cnt = torch.zeros(c.shape[:2], dtype=c.dtype).scatter_add_(1, a, torch.ones_like(a, dtype=c.dtype))
            c = torch.where((cnt > 0)[..., None], sums / cnt.clamp(min=1)[..., None], c)
        out.append(c)
    return torch.cat(out, 0)


_CB_CACHE: dict = {}


def codebooks(cfg: Workload, layer: int, device="cpu"):
    """(cb8 [Hkv][G][256][8], cb4 [Hkv][G][16][8]) float32 codebooks for one
    layer, fitted on the CPU and moved to `device`."""
    key = (cfg, layer)
    if key not in _CB_CACHE:
        H, D = cfg.num_kv_heads, cfg.head_dim
        G = D // 8
        n = cfg.codebook_samples
        s = torch.from_numpy(channel_scales(cfg, layer, "key")).double()
        z = torch.from_numpy(_rng(cfg.seed, layer, "cb-samples").standard_normal((H, n, D)))
        k = (z * s[:, None, :]).to(torch.float16).double()
        u = (k / k.norm(dim=-1, keepdim=True).clamp(min=1e-300)).float()
        x = u.reshape(H, n, G, 8).permute(0, 2, 1, 3).reshape(H * G, n, 8).contiguous()
        perm = torch.from_numpy(_rng(cfg.seed, layer, "cb-init").permutation(n))
        cb8 = _lloyd(x, 256, cfg.lloyd_iters, perm).reshape(H, G, 256, 8)
        cb4 = _lloyd(x, 16, cfg.lloyd_iters, perm).reshape(H, G, 16, 8)
        if len(_CB_CACHE) > 64:
            _CB_CACHE.clear()
        _CB_CACHE[key] = (cb8.contiguous(), cb4.contiguous())
    cb8, cb4 = _CB_CACHE[key]
    return cb8.to(device), cb4.to(device)


def place_perm(cfg: Workload, layer: int, n_pages: int, stream: str = "place"):
    """Physical placement order of a pack call's pages: identity (None) or a
    seeded random permutation for workloads with a permuted pool."""
    if not cfg.permuted_pool:
        return None
    return _rng(cfg.seed, layer, stream).permutation(n_pages).astype(np.uint32)
