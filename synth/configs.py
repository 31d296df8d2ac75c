"""Workload shapes (data only).

Five workloads, smallest first.  The shapes restate the serving pattern of the
zhiding.cn recsys-examples article, section "语义ID生成式推荐专用推理框架"
(long context of thousands of tokens, 2-3 semantic-ID tokens, beam 128/256,
Qwen3-1.7B at context 1,000 and 5,000 with beam 256 and 3 output tokens), and
of the paper-daily summary "Advancing Generative Recommendation Inference",
section "Performance" (prompt 2,000 tokens, 5 generated tokens, beam 30) with
its "Limitations" section (concurrency cap 64, unique prompts, no KV reuse).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Tuple, Union


@dataclass(frozen=True)
class Config:
    name: str
    cfg_id: int                      # enters every Philox key
    dtype: str                       # "f32" or "bf16": context K/V and token tables
    n_requests: int
    n_layers: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ctx_len: Union[int, Tuple[int, int]]          # fixed, or uniform integer range [lo, hi]
    beam_width: Union[int, Tuple[int, ...]]       # fixed, or choices drawn uniformly
    n_levels: int                    # semantic-ID length = decode steps
    codebook: int                    # codes per level
    n_items: int
    item_dist: str = "uniform"       # "uniform" or "zipf"
    zipf_a: float = 1.1
    waves: int = 1                   # admission waves (continuous batching)
    seed: int = 0
    shapes: Tuple[Tuple[int, int], ...] = ()   # explicit (ctx_len, beam_width) per request
    # exact power-of-two scalings of the drawn values (large query and key norms, as a trained
    # model's activations have them): queries (q_last and the query table) by 2^q_scale_log2,
    # context keys by 2^k_scale_log2, the fed-back tokens' keys by 2^own_k_scale_log2
    q_scale_log2: int = 0
    k_scale_log2: int = 0
    own_k_scale_log2: int = 0
    # "tables": q/k/v of a fed-back code from per-(layer, level, code) tables, layers summed;
    # "chain": a pre-norm decoder layer chain (RMSNorm, q/k/v/o projections, SwiGLU MLP of width
    # `intermediate`) whose layer l+1 reads layer l's output
    model: str = "tables"
    intermediate: int = 0
    notes: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def hidden(self) -> int:
        return self.n_q_heads * self.head_dim


CONFIGS = {
    c.name: c
    for c in [
        Config("tiny_f32", 1, "f32", 1, 1, 4, 2, 64, 64, 4, 3, 16, 200,
               notes="fp32 parity case; q/k/v tables and w_sid drawn with default_rng(0)"),
        Config("ctx1k_beam256", 2, "bf16", 1, 1, 16, 8, 128, 1000, 256, 3, 256, 1_000_000,
               notes="one Qwen3-1.7B-shaped layer, one request"),
        Config("ctx5k_beam256_r8", 3, "bf16", 8, 28, 16, 8, 128, 5000, 256, 3, 256, 1_000_000,
               notes="all 28 layers, 8 concurrent requests with distinct contexts"),
        Config("ctx2k_beam30_r64", 4, "bf16", 64, 28, 16, 8, 128, 2000, 30, 5, 256, 2_000_000,
               item_dist="zipf", notes="wide-request, narrow-beam mix"),
        Config("ragged_r128", 5, "bf16", 128, 28, 16, 8, 128, (500, 8000), (32, 128, 256), 3, 256,
               1_000_000, waves=4, notes="continuous-batching ragged mix in 4 admission waves"),
        Config("chain_ctx5k_beam256_r8", 6, "bf16", 8, 28, 16, 8, 128, 5000, 256, 3, 256, 1_000_000,
               model="chain", intermediate=6144,
               notes="the headline shapes with a Qwen3-1.7B-shaped layer chain (hidden 2048, MLP 6144)"),
    ]
}

HEADLINE = "ctx5k_beam256_r8"


def get_config(name: str, **overrides) -> Config:
    """Return a named config, optionally with fields replaced (smaller test variants)."""
    base = CONFIGS[name]
    if not overrides:
        return base
    d = {f: getattr(base, f) for f in base.__dataclass_fields__}
    d.update(overrides)
    return Config(**d)
