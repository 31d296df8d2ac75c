"""BeamEngine: holds the torch-owned device buffers of one gr_engine and forwards to the C ABI.

PyTorch only allocates device memory and supplies the stream; every step of
the decode runs in libgr_beam.so.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import _lib as G


def _torch():
    import torch
    return torch


def to_device(arr: np.ndarray, device="cuda"):
    """numpy -> torch device tensor; uint16 arrays are bf16 bit patterns and become bfloat16."""
    torch = _torch()
    a = np.ascontiguousarray(arr)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


class BeamEngine:
    """One engine: model tables, item trie, workspace.

    tok_q/tok_k/tok_v/w_sid are numpy arrays (bf16 bit patterns as uint16, or float32) or torch
    device tensors; items is a [n_items][n_levels] integer array.  chain: the layer-chain model's
    weights, a dict (embed, wq, wk, wv, wo, wg, wu, wd as bf16 [..][out][in], g_attn, g_mlp,
    g_final float32; numpy or torch device tensors) with "intermediate" and "eps"; the token
    tables are then unused (None).  w_label: the label head [Hq*d][n_labels] float32 (numpy or a
    torch device tensor); the token tables then hold n_levels levels, the last one for a
    candidate's last code."""

    def __init__(self, *, tok_q, tok_k, tok_v, w_sid, items, n_layers: int, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, dtype: str = "bf16", norm: str = "valid", max_requests: int = 1,
                 max_beam_width: int = 256, max_ctx_tokens: int = 0, max_splits: int = 0,
                 debug_attn: bool = False, max_layers_per_launch: int = 0, per_layer: bool = False,
                 chain=None, w_label=None, graph=False, device="cuda"):
        torch = _torch()
        self.device = device
        self.dtype = dtype
        conv = lambda x: x if (x is None or isinstance(x, torch.Tensor)) else to_device(x, device)
        self.tok_q, self.tok_k, self.tok_v = conv(tok_q), conv(tok_k), conv(tok_v)
        self._chain = None
        self._chain_I = chain["intermediate"] if chain is not None else 0
        chain_desc = None
        if chain is not None:
            self._chain = {k: conv(v) for k, v in chain.items() if k not in ("intermediate", "eps")}
            c = self._chain
            chain_desc = G.gr_chain_desc(int(chain["intermediate"]), float(chain["eps"]),
                                         *(c[k].data_ptr() for k in ("embed", "wq", "wk", "wv", "wo", "wg", "wu",
                                                                     "wd", "g_attn", "g_mlp", "g_final")))
        ptr = lambda t: t.data_ptr() if t is not None else None
        self.w_label, label_desc = None, None
        if w_label is not None:
            self.w_label = w_label if isinstance(w_label, torch.Tensor) else conv(np.asarray(w_label, dtype=np.float32))
            label_desc = G.gr_label_desc(int(self.w_label.shape[1]), self.w_label.data_ptr())
        self.w_sid = conv(np.asarray(w_sid, dtype=np.float32)) if not isinstance(w_sid, torch.Tensor) else w_sid
        self.n_layers, self.n_levels, self.V = int(n_layers), int(self.w_sid.shape[0]), int(self.w_sid.shape[2])
        self.Hq, self.Hkv, self.d = n_q_heads, n_kv_heads, head_dim
        desc = G.gr_model_desc(self.n_layers, n_q_heads, n_kv_heads, head_dim, self.n_levels, self.V,
                               G.GR_DTYPE_BF16 if dtype == "bf16" else G.GR_DTYPE_F32,
                               G.GR_NORM_VALID if norm == "valid" else G.GR_NORM_FULL,
                               ptr(self.tok_q), ptr(self.tok_k), ptr(self.tok_v), self.w_sid.data_ptr(),
                               C.pointer(chain_desc) if chain_desc is not None else None,
                               C.pointer(label_desc) if label_desc is not None else None)
        opts = G.gr_engine_opts(max_requests, max_beam_width, max_ctx_tokens, max_splits,
                                (G.GR_ENGINE_DEBUG_ATTN if debug_attn else 0) |
                                (G.GR_ENGINE_PER_LAYER if per_layer else 0) | (G.GR_ENGINE_GRAPH if graph else 0),
                                max_layers_per_launch)
        self.max_beam_width = max_beam_width
        self.eng = G.gr_engine_create(desc, np.asarray(items), opts)
        self.ws_bytes = G.gr_engine_workspace_bytes(self.eng)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        G.gr_engine_bind_workspace(self.eng, self.ws, self.ws_bytes, self.stream)
        self._keep = {}

    @property
    def stream(self) -> int:
        return _torch().cuda.current_stream().cuda_stream

    def trie_nodes(self, level: int) -> int:
        return G.gr_engine_trie_nodes(self.eng, level)

    def load(self, rid: int, k, v, q_last, beam_width: int, adopt: bool = False, ctx_len: int | None = None):
        """k, v: torch device tensors, [L][N][Hkv][d] (copy) or native K / V^T (adopt)."""
        n = ctx_len if ctx_len is not None else (k.shape[1] if not adopt else None)
        if n is None:
            raise ValueError("ctx_len is required with adopt=True")
        G.gr_ctx_kv_load(self.eng, rid, n, beam_width, k, v, q_last, G.GR_LOAD_ADOPT if adopt else 0, self.stream)
        if adopt:
            self._keep[rid] = (k, v)

    def set_prefill(self, tok_q, tok_k, tok_v, proj=None, w_q=None, w_k=None, w_v=None):
        """Context-token tables [L][Vc][H][d] (model dtype) and, for a soft token, the projection
        proj [user_dim][embed_dim] and w_q/w_k/w_v [L][embed_dim][H*d], float32.  numpy arrays are
        uploaded; torch device tensors are used in place.  The engine keeps them alive."""
        torch = _torch()
        dev = (lambda x: x) if isinstance(tok_k, torch.Tensor) else (lambda x: to_device(x, self.device))
        tabs = [dev(t) for t in (tok_q, tok_k, tok_v)]
        soft = []
        if proj is not None:
            f32 = lambda x: x if isinstance(x, torch.Tensor) else to_device(np.asarray(x, dtype=np.float32), self.device)
            soft = [f32(x) for x in (proj, w_q, w_k, w_v)]
        desc = G.gr_prefill_desc(int(tabs[1].shape[1]), *(t.data_ptr() for t in tabs),
                                 int(soft[0].shape[0]) if soft else 0, int(soft[0].shape[1]) if soft else 0,
                                 *((x.data_ptr() for x in soft) if soft else (None,) * 4))
        G.gr_engine_set_prefill(self.eng, desc)
        self._keep_pf = (tabs, soft)

    def prefill(self, rid: int, tokens, beam_width: int, soft_pos: int = -1, user_vec=None, k_native=None,
                vt_native=None, q_last_out=None):
        """Admit rid with its context made from token ids (host int array), one position
        optionally a soft token of user_vec (device float32 [user_dim]); with k_native/vt_native
        (device, native layout) the context goes there and the request keeps them."""
        G.gr_ctx_prefill(self.eng, rid, tokens, soft_pos, user_vec, beam_width, k_native, vt_native, q_last_out,
                         self.stream)
        if k_native is not None:
            self._keep[rid] = (k_native, vt_native)

    def prefill_noalloc(self, rid: int, tokens_dev, beam_width: int, soft_pos: int = -1, user_vec=None,
                        k_native=None, vt_native=None, q_last_out=None):
        """prefill() with the token ids in device memory (torch int32 tensor) and no allocation by
        the library (gr_ctx_prefill_noalloc)."""
        G.gr_ctx_prefill_noalloc(self.eng, rid, tokens_dev, int(tokens_dev.shape[0]), soft_pos, user_vec, beam_width,
                                 k_native, vt_native, q_last_out, self.stream)
        if k_native is not None:
            self._keep[rid] = (k_native, vt_native)

    def step(self, rids):
        G.gr_beam_step(self.eng, rids, self.stream)

    def beams(self, rid: int):
        return G.gr_beams_get(self.eng, rid, self.max_beam_width, self.n_levels, self.stream)

    def beams_batch(self, rids):
        return G.gr_beams_get_batch(self.eng, rids, self.max_beam_width, self.n_levels, self.stream)

    @property
    def result_bytes(self) -> int:
        """Bytes of one request's record in a beams_batch_async buffer."""
        return G.gr_beams_result_bytes(self.eng)

    def result_buffer(self, n: int):
        """Pinned host buffer for n records of beams_batch_async."""
        return _torch().empty(max(n, 1) * self.result_bytes, dtype=_torch().uint8, pin_memory=True)

    def beams_batch_async(self, rids, buf):
        """Enqueue the gather and copy of rids' beams into pinned `buf` on the current stream and
        return an event recorded after it; unpack(buf, i) once the event has completed."""
        n = len(rids)
        if buf.numel() < n * self.result_bytes or not buf.is_pinned():
            raise ValueError("buf must be pinned host memory of len(rids) * result_bytes bytes")
        G.gr_beams_get_batch_async(self.eng, rids, buf.data_ptr(), self.stream)
        ev = _torch().cuda.Event()
        ev.record()
        return ev

    def unpack(self, buf, i: int):
        """(codes [n][n_levels], scores [n]) of record i of a completed beams_batch_async."""
        return G.gr_beams_unpack(self.eng, buf.data_ptr(), i, self.max_beam_width, self.n_levels)

    def score_items(self, rid: int, items):
        """Log-probability of each given item (its code tuple) over the request's context."""
        return G.gr_score_items(self.eng, rid, items, self.stream)

    def score_items_batch(self, rids, items):
        """[len(rids)][n] log-probabilities; items [len(rids)][n][n_levels]."""
        return G.gr_score_items_batch(self.eng, rids, items, self.stream)

    def score_items_labels(self, rids, items):
        """Item log-likelihoods [len(rids)][n] and label log-probabilities [len(rids)][n][n_labels]
        of items [len(rids)][n][n_levels] (an engine with a label head)."""
        return G.gr_score_items_labels(self.eng, rids, items, int(self.w_label.shape[1]), self.stream)

    def reset(self, rid: int):
        G.gr_request_reset(self.eng, rid, self.stream)

    def reset_batch(self, rids):
        G.gr_request_reset_batch(self.eng, rids, self.stream)

    def release(self, rid: int):
        G.gr_request_release(self.eng, rid)
        self._keep.pop(rid, None)

    def state(self, rid: int):
        return G.gr_debug_beam_state(self.eng, rid, self.max_beam_width, self.n_levels, self.stream)

    def path(self, rid: int):
        return G.gr_debug_beam_path(self.eng, rid, self.max_beam_width, self.n_levels, self.stream)

    def chain_rows(self, rid: int, layer: int, which: int):
        """Rows of the layer chain's last step (debug engines): which = G.GR_CHAIN_*."""
        width = int(self._chain_I) if which == G.GR_CHAIN_ACT else self.Hq * self.d
        return G.gr_debug_chain_rows(self.eng, rid, layer, which, self.max_beam_width, width, self.stream)

    def hidden(self, rid: int):
        return G.gr_debug_hidden(self.eng, rid, self.max_beam_width, self.Hq * self.d, self.V, self.stream)

    def attn_out(self, rid: int, layer: int):
        return G.gr_debug_attn_out(self.eng, rid, layer, self.max_beam_width, self.Hq, self.d, self.stream)

    def close(self):
        if getattr(self, "eng", None):
            G.gr_engine_destroy(self.eng)
            self.eng = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class Scheduler:
    """Continuous batching over one BeamEngine (gr_sched_*): FIFO admission up to max_active
    decoding requests, one batched step per advance(), results one step later."""

    def __init__(self, engine: BeamEngine, max_active: int):
        self.engine = engine
        self.sched = G.gr_sched_create(engine.eng, max_active, engine.stream)
        self._keep = {}

    def submit(self, rid: int, k, v, q_last, beam_width: int, ctx_len: int | None = None, adopt: bool = False):
        """Queue a request (k, v, q_last as for BeamEngine.load; kept alive until admitted)."""
        n = ctx_len if ctx_len is not None else k.shape[1]
        G.gr_sched_submit(self.sched, rid, n, beam_width, k, v, q_last, G.GR_LOAD_ADOPT if adopt else 0)
        self._keep[rid] = (k, v, q_last)

    def advance(self) -> int:
        """One scheduling round; returns the number of results that became available."""
        return G.gr_sched_advance(self.sched)

    def flush(self) -> int:
        return G.gr_sched_flush(self.sched)

    def completed(self, capacity: int = 1 << 16):
        return G.gr_sched_completed(self.sched, capacity)

    def result(self, rid: int):
        """(codes [n][n_levels], scores [n]) of a finished request, taken out of the store."""
        out = G.gr_sched_result(self.sched, rid, self.engine.max_beam_width, self.engine.n_levels)
        self._keep.pop(rid, None)
        return out

    def counts(self):
        return G.gr_sched_counts(self.sched)

    def close(self):
        if getattr(self, "sched", None):
            G.gr_sched_destroy(self.sched)
            self.sched = None
        self._keep.clear()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
