"""Seeded synthetic inputs for the semantic-ID beam-decode step.

This package only draws numbers. It holds none of the decode step's
arithmetic (no attention, no log-softmax, no selection): it produces the
context K/V, the per-(level, code) query/key/value tables that stand in for
the model's QKV projection of a fed-back code, the codebook projection
``w_sid``, and the set of valid items (code tuples).  Both the CPU oracle and
the GPU path consume what it returns; neither is imported here.

Workload shapes follow the serving pattern described in the zhiding.cn
article on NVIDIA recsys-examples, section "语义ID生成式推荐专用推理框架"
(semantic-ID generative-recommendation inference framework): thousands of
context tokens, two to three decoded semantic-ID tokens, beam width 128/256,
Qwen3-1.7B attention shape (16 query heads, 8 KV heads, head_dim 128), and the
paper-daily summary "Advancing Generative Recommendation Inference",
section "Performance" (prompt 2000, 5 generated tokens, beam 30).

Value recipes
-------------
* bf16 tensors: a Philox4x64 counter stream (numpy ``Philox`` keyed per block)
  gives uniform 16-bit indices ``i``; the value is ``bf16(Phi^-1((i+0.5)/65536))``,
  a discretised N(0,1) that is exact in bf16.  Every (config, tensor, request,
  layer) block has its own key, so any block can be regenerated alone.
* fp32 tensors (the tiny config and every ``w_sid``): ``numpy.random.default_rng``
  normal draws, in a fixed order.
* items: distinct code tuples, big-endian (level 0 is the most significant
  code).  Uniform configs draw without replacement from all V**levels tuples;
  the Zipf config draws each level's code by a Zipf(1.1) rank mapped through a
  per-level seeded permutation, de-duplicates, and keeps the first distinct
  tuples in draw order.
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    BF16_NORMAL_TABLE,
    CHAIN_MATS,
    bf16_bits_to_f32,
    chain_embed,
    chain_gains,
    chain_matrix,
    chain_scale,
    chain_shapes,
    chain_weights,
    x_last,
    ctx_kv_block,
    items,
    label_token_tables,
    prefill_tables,
    prefill_tokens,
    q_last,
    request_shapes,
    soft_token_weights,
    token_tables,
    token_tables_with_labels,
    user_vector,
    w_label,
    w_sid,
)
