"""Engines and request inputs for the synthetic workloads (tests, bench.py and smoke()).

Builds a BeamEngine from a workload description of the seeded input generators (`synth`) and
puts a request's context into device memory.  Argument marshalling and data placement only:
every step of the decode runs in libgr_beam.so.
"""
from __future__ import annotations

import numpy as np


def make_engine(cfg, *, max_requests=None, max_splits=0, debug_attn=False, norm="valid", max_ctx_tokens=None,
                max_beam_width=None, max_layers_per_launch=0, per_layer=False, n_labels=0, graph=False):
    """An engine for a synthetic workload; n_labels > 0 adds a label head (and the label level of
    the token tables) for candidate scoring by label tokens."""
    import synth

    from .engine import BeamEngine
    from ._lib import lib
    chain = None
    if cfg.model == "chain":
        tq = tk = tv = None
        chain = chain_weights(cfg)
    elif n_labels > 0:
        tq, tk, tv = synth.token_tables_with_labels(cfg)
    else:
        tq, tk, tv = synth.token_tables(cfg)
    shapes = synth.request_shapes(cfg)
    R = cfg.n_requests if max_requests is None else max_requests
    if max_ctx_tokens is None:
        max_ctx_tokens = sum(lib().gr_ctx_padded_len(n) for n, _ in shapes[:R])
    W = max(w for _, w in shapes) if max_beam_width is None else max_beam_width
    return BeamEngine(tok_q=tq, tok_k=tk, tok_v=tv, w_sid=synth.w_sid(cfg), items=synth.items(cfg),
                      n_layers=cfg.n_layers, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                      head_dim=cfg.head_dim, dtype=cfg.dtype, norm=norm, max_requests=R,
                      max_beam_width=W, max_ctx_tokens=max_ctx_tokens, max_splits=max_splits,
                      debug_attn=debug_attn, max_layers_per_launch=max_layers_per_launch, per_layer=per_layer,
                      chain=chain, w_label=synth.w_label(cfg, n_labels) if n_labels > 0 else None, graph=graph)


def chain_weights(cfg, device="cuda", eps: float = 1e-6) -> dict:
    """The layer chain's weights of a chain workload as device tensors (drawn on the device for
    large models), with its MLP width and norm epsilon."""
    import synth
    n_params = cfg.n_layers * sum(r * c for r, c in synth.chain_shapes(cfg).values())
    if n_params > (1 << 26) and str(device).startswith("cuda"):
        from synth import device as synth_device
        w = synth_device.chain_weights(cfg, device)
    else:
        w = synth.chain_weights(cfg)
    return {**w, "intermediate": cfg.intermediate, "eps": eps}


def request_tensors(cfg, r: int, device="cuda", host=False):
    """Context K, V [L][N][Hkv][d] and q_last [L][Hq][d] of request r as device tensors.

    bf16 workloads are generated on the device (synth.device: the host generators' values)
    unless `host`; fp32 ones on the host."""
    import synth

    from .engine import to_device
    if cfg.dtype == "bf16" and not host and str(device).startswith("cuda"):
        from synth import device as synth_device
        k, v, q = synth_device.request_tensors(cfg, r, device)
        if cfg.model == "chain":   # the last context token's input vector instead of per-layer queries
            q = to_device(synth.x_last(cfg, r), device)
        return k, v, q
    ks, vs = [], []
    for l in range(cfg.n_layers):
        k, v = synth.ctx_kv_block(cfg, r, l)
        ks.append(k)
        vs.append(v)
    q = synth.x_last(cfg, r) if cfg.model == "chain" else synth.q_last(cfg, r)
    return to_device(np.stack(ks), device), to_device(np.stack(vs), device), to_device(q, device)


def native_layout(k, v):
    """[L][N][Hkv][d] -> (K [L][Hkv][Np][d], V^T [L][Hkv][d][Np]) zero-padded (data placement for
    GR_LOAD_ADOPT)."""
    import torch
    L, N, Hkv, d = k.shape
    Np = (N + 63) // 64 * 64
    kn = torch.zeros((L, Hkv, Np, d), dtype=k.dtype, device=k.device)
    vn = torch.zeros((L, Hkv, d, Np), dtype=v.dtype, device=v.device)
    kn[:, :, :N, :] = k.permute(0, 2, 1, 3)
    vn[:, :, :, :N] = v.permute(0, 2, 3, 1)
    return kn.contiguous(), vn.contiguous(), N


def load_request(eng, cfg, r: int, rid: int | None = None, adopt=False):
    import synth
    k, v, q = request_tensors(cfg, r)
    N, W = synth.request_shapes(cfg)[r]
    rid = r if rid is None else rid
    if adopt:
        kn, vn, _ = native_layout(k, v)
        eng.load(rid, kn, vn, q, W, adopt=True, ctx_len=N)
    else:
        eng.load(rid, k, v, q, W)
    return rid
