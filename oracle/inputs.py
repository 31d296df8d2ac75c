"""The oracle's view of the seeded synthetic workloads (test infrastructure only).

Builds the float64 model, the valid-prefix sets and per-request contexts from the input
generators in `synth` (the only module the oracle and the HIP path both use)."""
from __future__ import annotations

import functools

from . import beam
from .beam import Model, PrefixSet, Request


@functools.lru_cache(maxsize=8)
def model_for(cfg) -> Model:
    import synth
    tq, tk, tv = synth.token_tables(cfg)
    return Model.from_arrays(tq, tk, tv, synth.w_sid(cfg))


@functools.lru_cache(maxsize=8)
def label_model_for(cfg) -> Model:
    """The model with the label level's token tables appended (candidate scoring by labels)."""
    import synth
    tq, tk, tv = synth.token_tables_with_labels(cfg)
    return Model.from_arrays(tq, tk, tv, synth.w_sid(cfg))


@functools.lru_cache(maxsize=8)
def prefixes_for(cfg) -> PrefixSet:
    import synth
    return PrefixSet(synth.items(cfg), cfg.codebook)


def request_for(cfg, r: int, cache: bool = True) -> Request:
    """The oracle's view of request r; context blocks are regenerated per layer on demand."""
    import synth
    store = {}

    def ctx(l):
        if cache and l in store:
            return store[l]
        k, v = synth.ctx_kv_block(cfg, r, l)
        kv = (beam.as_f64(k), beam.as_f64(v))
        if cache:
            store[l] = kv
        return kv

    return Request(ctx=ctx, q_last=beam.as_f64(synth.q_last(cfg, r)))


@functools.lru_cache(maxsize=4)
def chain_model_for(cfg):
    """The layer-chain model of a chain workload (every layer's weights on the host)."""
    import synth

    from .chain import ChainModel
    return ChainModel.from_arrays(synth.chain_weights(cfg), synth.w_sid(cfg), cfg.n_q_heads, cfg.n_kv_heads)


def chain_request_for(cfg, r: int, cache: bool = True):
    """The chain oracle's view of request r: the context blocks and the last token's input."""
    import synth

    from .chain import ChainRequest
    base = request_for(cfg, r, cache)
    return ChainRequest(ctx=base.ctx, x_last=synth.x_last(cfg, r).astype("float64"))

