"""Builds oracle inputs from the seeded generators (test side only)."""
from __future__ import annotations

import functools

import numpy as np

import oracle
import synth


@functools.lru_cache(maxsize=8)
def model_for(cfg) -> "oracle.Model":
    tq, tk, tv = synth.token_tables(cfg)
    return oracle.Model.from_arrays(tq, tk, tv, synth.w_sid(cfg))


@functools.lru_cache(maxsize=8)
def prefixes_for(cfg) -> "oracle.PrefixSet":
    return oracle.PrefixSet(synth.items(cfg), cfg.codebook)


def request_for(cfg, r: int, cache: bool = True) -> "oracle.Request":
    """The oracle's view of request r; context blocks are regenerated per layer on demand."""
    store = {}

    def ctx(l):
        if cache and l in store:
            return store[l]
        k, v = synth.ctx_kv_block(cfg, r, l)
        kv = (oracle.beam.as_f64(k), oracle.beam.as_f64(v))
        if cache:
            store[l] = kv
        return kv

    return oracle.Request(ctx=ctx, q_last=oracle.beam.as_f64(synth.q_last(cfg, r)))


def dict_trie(items: np.ndarray):
    """Dict-of-sets trie: prefix tuple -> set of next codes (independent of PrefixSet)."""
    t = {}
    for it in items.tolist():
        for s in range(len(it)):
            t.setdefault(tuple(it[:s]), set()).add(it[s])
    return t
