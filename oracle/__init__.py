"""CPU oracle for the semantic-ID beam-decode step.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library under
``semantic_id_beam_amd/`` never imports it, and it imports nothing from there:
the two share no code.  Everything here is plain numpy float64, written for a
reader to check against the pages by eye, not for speed.

What it computes (one request, one beam-search decode):

* Semantic-ID beam search: every item is a short tuple of codes generated one
  code per step; the search keeps the best prefixes, expands each by one code,
  prunes, and returns every surviving complete code tuple (paper-daily
  "Advancing Generative Recommendation Inference", section "Background";
  zhiding.cn recsys-examples article, section "语义ID" on beam search
  producing several semantic IDs at once).
* Each beam is recomputed as an independent full sequence -- the shared
  context followed by the beam's own decoded tokens -- exactly the form the
  ContextKV / BeamKV / BeamPath split of the zhiding.cn article (section
  "语义ID生成式推荐专用推理框架") is built to avoid.  Attention, logits,
  constrained log-softmax and an exhaustive sort, nothing shared across beams.
* Item-constrained generation (same section): only codes that extend a
  valid item prefix are candidates.
* Candidate scoring (paper-daily article, section "Background": given
  candidates are ranked by the model): an item's log-probability is the sum
  of its per-level constrained log-probabilities at its own prefixes; and by
  label tokens (sections "Background" and "Scoring many candidates at once"):
  the label log-probabilities read from each candidate's last token, the
  candidate seeing the context and itself only (``label_scores``).

Readings where the pages are silent (each is a choice, see ``beam.py``):
query of step 0 is the last context token's query; a fed-back code's q/k/v
come from per-(layer, level, code) tables; layer outputs are summed into a
head-major hidden vector with no other layers; scale 1/sqrt(d); contiguous
GQA (kv = hq // g); log-softmax normalised over the valid codes (R2) or the
whole codebook (R1); ties broken by flat index j*V + c ascending; the beam
count after a step is min(W, number of valid candidates).

* A real layer chain (``chain.py``): a Qwen3-1.7B-shaped pre-norm decoder whose layer l+1
  reads layer l's output (RMSNorm, q/k/v/o projections, SwiGLU MLP, final RMSNorm), with the
  bf16 rounding points of its projections' inputs stated as part of the model.

* Prefill (``prefill.py``): the context K/V and first query from context
  token ids, one position optionally a soft token projected from a user
  vector (paper-daily article, section "Getting the user vector into the
  prompt: three approaches").

Parity status per function: every function in ``beam.py`` and ``prefill.py`` is pinned by tests
in ``tests/test_oracle.py`` and ``tests/test_oracle_prefill.py`` (closed forms, a hand-derived worked example,
library cross-checks, brute-force enumeration, greedy special case,
invariants).  No function is "parity unpinned".
"""
from .beam import (  # noqa: F401
    Model,
    PrefixSet,
    Request,
    attend,
    beam_hidden,
    beam_layer_output,
    beam_search,
    codebook_logits,
    constrained_log_softmax,
    label_scores,
    score_items,
    select_topk,
    step_candidates,
)
from .prefill import prefill_context, soft_embedding, soft_qkv  # noqa: F401
from .chain import (  # noqa: F401
    ChainModel,
    ChainRequest,
    beam_chain,
    bf16_round,
    chain_hidden,
    chain_layer_outputs,
    rms_norm,
    silu,
)
