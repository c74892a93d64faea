"""Workload table for the ADA decode path, and the byte-budget -> tier-mix rule.

Seven seeded synthetic workloads stand in for the pages' evaluation (three
instruction-tuned LLMs at 8K/32K/128K contexts on long-document, multi-hop QA
and agent-trajectory suites; gist.science technical summary of SPHERICAL KV,
section 4).  No dataset or model weight is used: only shapes, lengths and the
value distributions below.  Workloads 1-5 use the Llama-3-8B attention shape;
6 and 7 take the attention shapes of the other two models the pages name
(Qwen2.5-14B: 40 query / 8 KV heads of 128 dims; gpt-oss-20b: 64 query / 8
KV heads of 64 dims).  Those shapes come from the models' public
configurations, not from the pages.  Tier mixes are cumulative basis points
(fp16, fp16 + 8-bit, fp16 + 8-bit + 4-bit); the rest is dropped.
"""
from __future__ import annotations

from dataclasses import dataclass, field

# Bytes one retained token-head occupies in a full page, by tier, for D = 128
# (fp16 keys 8192 B, 8-bit codes 4480 B, 4-bit codes 2304 B per 16-slot page).
TOKEN_BYTES_D128 = (512, 280, 144)
DENSE_TOKEN_BYTES_D128 = 512  # bf16 K + bf16 V


@dataclass(frozen=True)
class Workload:
    number: int
    name: str
    num_seqs: int
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    seq_len: int | None          # fixed length, or None for drawn lengths
    len_range: tuple[int, int] | None = None
    tier_cum_bp: tuple[int, int, int] | None = None  # fixed mix for every sequence
    budget_range_bp: tuple[int, int] | None = None   # drawn byte budget per sequence
    budget_bp: int = 6000        # fixed byte budget (basis points of dense) for the budget solver
    key_outliers: bool = True    # 1% of channels at 8x
    value_scaled: bool = False   # values also get lognormal channel scales
    permuted_pool: bool = False  # pages placed in a seeded random order
    append_tokens: int = 0       # tokens appended through encode + pack per seq/layer
    codebook_samples: int = 4096
    lloyd_iters: int = 10
    page_size: int = 16

    @property
    def seed(self) -> int:
        return 1000 + self.number

    @property
    def gqa(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def sigma(self) -> float:
        return 1.0 / float(self.head_dim) ** 0.5


WORKLOADS = {
    1: Workload(1, "tiny-mha-d64-t512", 1, 1, 4, 4, 64, 512,
                tier_cum_bp=(2500, 7500, 10000), key_outliers=False, value_scaled=True),
    2: Workload(2, "llama3-8b-shape-t32k", 1, 1, 32, 8, 128, 32768,
                tier_cum_bp=(1500, 6000, 8500)),
    3: Workload(3, "batch4-t128k-permuted-pool", 4, 1, 32, 8, 128, 131072,
                tier_cum_bp=(1000, 5000, 8000), permuted_pool=True),
    4: Workload(4, "ragged64-t4k-64k-budget40-80", 64, 1, 32, 8, 128, None,
                len_range=(4096, 65536), budget_range_bp=(4000, 8000), permuted_pool=True),
    5: Workload(5, "32layer-batch8-t128k", 8, 32, 32, 8, 128, 131072,
                tier_cum_bp=(1500, 6000, 8500), append_tokens=512),
    6: Workload(6, "qwen2.5-14b-shape-t32k", 1, 1, 40, 8, 128, 32768,
                tier_cum_bp=(1500, 6000, 8500)),
    7: Workload(7, "gpt-oss-20b-shape-t32k", 1, 1, 64, 8, 64, 32768,
                tier_cum_bp=(1500, 6000, 8500)),
}

# Endpoints of the budget rule: cumulative bp of two mixes whose stored bytes
# are 39.8% and 79.7% of a dense bf16 cache (D = 128 page sizes).
_MIX_LO = (1000, 4900, 7900)
_MIX_HI = (6100, 9000, 10000)


def mix_for_budget(budget_bp: int) -> tuple[int, int, int]:
    """Cumulative tier basis points whose full-page bytes stay within a byte
    budget of `budget_bp` / 10000 of the dense cache, for budgets in
    [4000, 8000].  The mix moves linearly from _MIX_LO to _MIX_HI as the budget
    goes from 40% to 80%; per-mille steps are floored so the stored fraction
    never exceeds the budget (partial last pages aside).

    The pages give the goal (keep and tier states under a strict budget,
    gist.science technical summary section 2.2) but no solver; this rule is a
    stand-in for the utility-driven allocator, not part of the decode path.
    """
    if not 4000 <= budget_bp <= 8000:
        raise ValueError("budget must be within [4000, 8000] basis points")
    t = (budget_bp - 4000) // 4  # per mille along the segment
    return tuple(lo + (hi - lo) * t // 1000 for lo, hi in zip(_MIX_LO, _MIX_HI))


def stored_fraction(cum_bp, token_bytes=TOKEN_BYTES_D128, dense=DENSE_TOKEN_BYTES_D128) -> float:
    """Full-page stored bytes of a mix as a fraction of the dense bf16 cache."""
    shares = (cum_bp[0], cum_bp[1] - cum_bp[0], cum_bp[2] - cum_bp[1])
    return sum(s * b for s, b in zip(shares, token_bytes)) / (10000.0 * dense)
