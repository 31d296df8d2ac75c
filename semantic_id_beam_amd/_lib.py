"""ctypes binding of libgr_beam.so (argument marshalling only).

Every function keeps the C name.  Tensors are passed as device pointers
(``tensor.data_ptr()``) or host numpy arrays; streams as ``hipStream_t``
handles (``torch.cuda.current_stream().cuda_stream``).  Every step of the
decode runs in the library's HIP kernels; nothing here computes.
A failing call raises GrError with the library's message.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# GR_BEAM_LIB_VARIANT=timed loads the wave-timeline measurement build instead (bench.py
# --wave-times starts a child process with it); nothing else selects it
LIB_PATH = os.path.join(_HERE, "libgr_beam_timed.so" if os.environ.get("GR_BEAM_LIB_VARIANT") == "timed"
                        else "libgr_beam.so")

GR_OK, GR_E_INVALID_ARG, GR_E_OUT_OF_MEMORY, GR_E_BAD_STATE, GR_E_NOT_FOUND, GR_E_DEVICE, GR_E_UNSUPPORTED = range(7)
GR_DTYPE_F32, GR_DTYPE_BF16 = 0, 1
GR_NORM_VALID, GR_NORM_FULL = 0, 1
GR_ENGINE_DEBUG_ATTN = 1
GR_ENGINE_PER_LAYER = 2
GR_ENGINE_GRAPH = 4
GR_LOAD_ADOPT = 1

STATUS_NAMES = {0: "GR_OK", 1: "GR_E_INVALID_ARG", 2: "GR_E_OUT_OF_MEMORY", 3: "GR_E_BAD_STATE",
                4: "GR_E_NOT_FOUND", 5: "GR_E_DEVICE", 6: "GR_E_UNSUPPORTED"}

#: every symbol include/gr_beam.h declares
EXPORTS = [
    "gr_engine_create", "gr_engine_workspace_bytes", "gr_engine_bind_workspace", "gr_engine_destroy",
    "gr_engine_trie_nodes", "gr_ctx_padded_len", "gr_ctx_kv_load", "gr_engine_set_prefill", "gr_ctx_prefill", "gr_ctx_prefill_noalloc",
    "gr_beam_step", "gr_beams_get",
    "gr_beams_get_batch", "gr_beams_get_batch_async", "gr_beams_result_bytes", "gr_beams_unpack",
    "gr_request_release", "gr_request_reset", "gr_request_reset_batch", "gr_last_error", "gr_topk_select", "gr_debug_beam_state", "gr_debug_beam_path",
    "gr_debug_hidden", "gr_debug_attn_out", "gr_engine_set_profiling", "gr_engine_profile_read",
    "gr_engine_profile_dispatches", "gr_engine_profile_reset", "gr_score_items", "gr_score_items_batch",
    "gr_sched_create", "gr_sched_destroy", "gr_sched_submit", "gr_sched_advance", "gr_sched_flush",
    "gr_sched_completed", "gr_sched_result", "gr_sched_counts", "gr_debug_chain_rows", "gr_score_items_labels",
    "gr_engine_graph_stats", "gr_engine_set_profiling_kinds", "gr_engine_set_profiling_stride",
    "gr_wave_times_select", "gr_wave_times_read",
]
GR_CHAIN_X_IN, GR_CHAIN_XN_ATTN, GR_CHAIN_Q, GR_CHAIN_O, GR_CHAIN_X_MID, GR_CHAIN_XN_MLP, GR_CHAIN_ACT, \
    GR_CHAIN_X_OUT = range(8)
GR_PROF_CTX_ATTN, GR_PROF_BEAM_MERGE, GR_PROF_LOGITS, GR_PROF_TOPK, GR_PROF_STEP, GR_PROF_GEMM, GR_PROF_NORM = range(7)


class GrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {msg}")
        self.status = status


class gr_chain_desc(C.Structure):
    _fields_ = [("intermediate", C.c_int32), ("rms_eps", C.c_float), ("embed", C.c_void_p), ("w_q", C.c_void_p),
                ("w_k", C.c_void_p), ("w_v", C.c_void_p), ("w_o", C.c_void_p), ("w_gate", C.c_void_p),
                ("w_up", C.c_void_p), ("w_down", C.c_void_p), ("g_attn", C.c_void_p), ("g_mlp", C.c_void_p),
                ("g_final", C.c_void_p)]


class gr_label_desc(C.Structure):
    _fields_ = [("n_labels", C.c_int32), ("w_label", C.c_void_p)]


class gr_model_desc(C.Structure):
    _fields_ = [("n_layers", C.c_int32), ("n_q_heads", C.c_int32), ("n_kv_heads", C.c_int32),
                ("head_dim", C.c_int32), ("n_levels", C.c_int32), ("codebook_size", C.c_int32),
                ("dtype", C.c_int32), ("norm", C.c_int32),
                ("tok_q", C.c_void_p), ("tok_k", C.c_void_p), ("tok_v", C.c_void_p), ("w_sid", C.c_void_p),
                ("chain", C.POINTER(gr_chain_desc)), ("label", C.POINTER(gr_label_desc))]


class gr_item_set(C.Structure):
    _fields_ = [("n_items", C.c_int64), ("codes", C.POINTER(C.c_int32))]


class gr_engine_opts(C.Structure):
    _fields_ = [("max_requests", C.c_int32), ("max_beam_width", C.c_int32), ("max_ctx_tokens", C.c_int64),
                ("max_splits", C.c_int32), ("flags", C.c_uint32), ("max_layers_per_launch", C.c_int32)]


class gr_prefill_desc(C.Structure):
    _fields_ = [("vocab", C.c_int32), ("tok_q", C.c_void_p), ("tok_k", C.c_void_p), ("tok_v", C.c_void_p),
                ("user_dim", C.c_int32), ("embed_dim", C.c_int32), ("proj", C.c_void_p), ("w_q", C.c_void_p),
                ("w_k", C.c_void_p), ("w_v", C.c_void_p)]


_lib = None


def lib() -> C.CDLL:
    """Load the HIP library (fails loudly if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    # Load torch first: its bundled HIP runtime then satisfies the library's
    # libamdhip64.so.7 dependency, so the library and torch share one runtime
    # (two runtimes in one process do not share devices or memory).
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with semantic_id_beam_amd/build.py "
                          "(or __graft_entry__.build())")
    L = C.CDLL(LIB_PATH)
    vp, i32, i64, u32, sz = C.c_void_p, C.c_int32, C.c_int64, C.c_uint32, C.c_size_t
    P = C.POINTER
    sig = {
        "gr_engine_create": (i32, [P(gr_model_desc), P(gr_item_set), P(gr_engine_opts), P(vp)]),
        "gr_engine_workspace_bytes": (sz, [vp]),
        "gr_engine_bind_workspace": (i32, [vp, vp, sz, vp]),
        "gr_engine_destroy": (i32, [vp]),
        "gr_engine_trie_nodes": (i32, [vp, i32, P(i64)]),
        "gr_ctx_padded_len": (i32, [i32]),
        "gr_ctx_kv_load": (i32, [vp, i64, i32, i32, vp, vp, vp, u32, vp]),
        "gr_engine_set_prefill": (i32, [vp, P(gr_prefill_desc)]),
        "gr_ctx_prefill": (i32, [vp, i64, vp, i32, i32, vp, i32, vp, vp, vp, vp]),
        "gr_ctx_prefill_noalloc": (i32, [vp, i64, vp, i32, i32, vp, i32, vp, vp, vp, vp]),
        "gr_beam_step": (i32, [vp, P(i64), i32, vp]),
        "gr_wave_times_select": (i32, [i32, i32]),
        "gr_wave_times_read": (i32, [P(i64), sz]),
        "gr_beams_get": (i32, [vp, i64, i32, vp, vp, P(i32), vp]),
        "gr_beams_get_batch": (i32, [vp, P(i64), i32, i32, vp, vp, vp, vp]),
        "gr_beams_get_batch_async": (i32, [vp, P(i64), i32, vp, vp]),
        "gr_beams_result_bytes": (sz, [vp]),
        "gr_beams_unpack": (i32, [vp, vp, i32, i32, vp, vp, P(i32)]),
        "gr_request_release": (i32, [vp, i64]),
        "gr_request_reset": (i32, [vp, i64, vp]),
        "gr_request_reset_batch": (i32, [vp, P(i64), i32, vp]),
        "gr_last_error": (C.c_char_p, []),
        "gr_topk_select": (i32, [vp, i32, i32, i32, vp, vp, vp, vp]),
        "gr_debug_beam_state": (i32, [vp, i64, i32, vp, vp, vp, P(i32), P(i32), vp]),
        "gr_debug_beam_path": (i32, [vp, i64, i32, vp, P(i32), vp]),
        "gr_debug_chain_rows": (i32, [vp, i64, i32, i32, i32, vp, P(i32), vp]),
        "gr_debug_hidden": (i32, [vp, i64, i32, vp, vp, P(i32), vp]),
        "gr_debug_attn_out": (i32, [vp, i64, i32, i32, vp, P(i32), vp]),
        "gr_engine_set_profiling": (i32, [vp, i32]),
        "gr_engine_profile_read": (i32, [vp, i32, i32, P(C.c_double), P(i64)]),
        "gr_engine_profile_dispatches": (i32, [vp, i32, i32, P(i64)]),
        "gr_score_items": (i32, [vp, i64, vp, i32, vp, vp]),
        "gr_score_items_batch": (i32, [vp, vp, i32, vp, i32, vp, vp]),
        "gr_score_items_labels": (i32, [vp, vp, i32, vp, i32, vp, vp, vp]),
        "gr_engine_profile_reset": (i32, [vp]),
        "gr_engine_graph_stats": (i32, [vp, vp, vp]),
        "gr_engine_set_profiling_kinds": (i32, [vp, C.c_uint32]),
        "gr_engine_set_profiling_stride": (i32, [vp, i32]),
        "gr_sched_create": (i32, [vp, i32, vp, P(vp)]),
        "gr_sched_destroy": (i32, [vp]),
        "gr_sched_submit": (i32, [vp, i64, i32, i32, vp, vp, vp, u32]),
        "gr_sched_advance": (i32, [vp, P(i32)]),
        "gr_sched_flush": (i32, [vp, P(i32)]),
        "gr_sched_completed": (i32, [vp, i32, vp, P(i32)]),
        "gr_sched_result": (i32, [vp, i64, i32, vp, vp, P(i32)]),
        "gr_sched_counts": (i32, [vp, P(i32), P(i32), P(i32), P(i64)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype, f.argtypes = res, args
    _lib = L
    return L


def _check(st: int):
    if st != GR_OK:
        raise GrError(st, lib().gr_last_error().decode())


def _ptr(x) -> int | None:
    """Device pointer of a torch tensor, an int, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _host(a: np.ndarray):
    return a.ctypes.data_as(C.c_void_p)


# ---------------------------------------------------------------- same names as the C ABI
def gr_engine_create(desc: gr_model_desc, items: np.ndarray, opts: gr_engine_opts) -> int:
    items = np.ascontiguousarray(items, dtype=np.int32)
    iset = gr_item_set(items.shape[0], items.ctypes.data_as(C.POINTER(C.c_int32)))
    out = C.c_void_p()
    _check(lib().gr_engine_create(C.byref(desc), C.byref(iset), C.byref(opts), C.byref(out)))
    return out.value


def gr_engine_workspace_bytes(eng: int) -> int:
    return lib().gr_engine_workspace_bytes(eng)


def gr_engine_bind_workspace(eng: int, ws, nbytes: int, stream: int = 0):
    _check(lib().gr_engine_bind_workspace(eng, _ptr(ws), nbytes, stream))


def gr_engine_destroy(eng: int):
    _check(lib().gr_engine_destroy(eng))


def gr_engine_trie_nodes(eng: int, level: int) -> int:
    n = C.c_int64()
    _check(lib().gr_engine_trie_nodes(eng, level, C.byref(n)))
    return n.value


def gr_ctx_padded_len(n: int) -> int:
    return lib().gr_ctx_padded_len(n)


def gr_ctx_kv_load(eng: int, rid: int, ctx_len: int, beam_width: int, k, v, q_last, flags: int = 0,
                   stream: int = 0):
    _check(lib().gr_ctx_kv_load(eng, rid, ctx_len, beam_width, _ptr(k), _ptr(v), _ptr(q_last), flags, stream))


def gr_engine_set_prefill(eng: int, desc: gr_prefill_desc):
    _check(lib().gr_engine_set_prefill(eng, C.byref(desc)))


def gr_ctx_prefill(eng: int, rid: int, tokens, soft_pos: int, user_vec, beam_width: int, k_native=None,
                   vt_native=None, q_last_out=None, stream: int = 0):
    """tokens: host int32 [N]; user_vec, k_native, vt_native, q_last_out: device pointers or None."""
    tok = np.ascontiguousarray(tokens, dtype=np.int32)
    _check(lib().gr_ctx_prefill(eng, rid, _host(tok), tok.shape[0], soft_pos, _ptr(user_vec), beam_width,
                                _ptr(k_native), _ptr(vt_native), _ptr(q_last_out), stream))


def gr_ctx_prefill_noalloc(eng: int, rid: int, tokens_dev, ctx_len: int, soft_pos: int, user_vec, beam_width: int,
                           k_native=None, vt_native=None, q_last_out=None, stream: int = 0):
    """tokens_dev: device int32 [ctx_len]; user_vec, k_native, vt_native, q_last_out: device pointers or None."""
    _check(lib().gr_ctx_prefill_noalloc(eng, rid, _ptr(tokens_dev), ctx_len, soft_pos, _ptr(user_vec), beam_width,
                                        _ptr(k_native), _ptr(vt_native), _ptr(q_last_out), stream))


def gr_beam_step(eng: int, request_ids, stream: int = 0):
    ids = np.ascontiguousarray(request_ids, dtype=np.int64)
    _check(lib().gr_beam_step(eng, ids.ctypes.data_as(C.POINTER(C.c_int64)), ids.shape[0], stream))


def gr_beams_get(eng: int, rid: int, capacity: int, n_levels: int, stream: int = 0):
    codes = np.zeros((max(capacity, 1), n_levels), dtype=np.int32)
    scores = np.zeros(max(capacity, 1), dtype=np.float32)
    n = C.c_int32()
    _check(lib().gr_beams_get(eng, rid, capacity, _host(codes), _host(scores), C.byref(n), stream))
    return codes[: n.value], scores[: n.value]


def gr_beams_get_batch(eng: int, request_ids, capacity: int, n_levels: int, stream: int = 0):
    """[(codes [n_i][n_levels], scores [n_i]) for each id], one synchronisation for all."""
    ids = np.ascontiguousarray(request_ids, dtype=np.int64)
    n = ids.shape[0]
    codes = np.zeros((n, max(capacity, 1), n_levels), dtype=np.int32)
    scores = np.zeros((n, max(capacity, 1)), dtype=np.float32)
    nb = np.zeros(n, dtype=np.int32)
    _check(lib().gr_beams_get_batch(eng, ids.ctypes.data_as(C.POINTER(C.c_int64)), n, capacity, _host(codes),
                                    _host(scores), _host(nb), stream))
    return [(codes[i, : nb[i]], scores[i, : nb[i]]) for i in range(n)]


def gr_beams_get_batch_async(eng: int, request_ids, out_host: int, stream: int = 0) -> None:
    """Enqueue the gather of each request's beams into records at out_host (caller-owned pinned
    host memory, n * gr_beams_result_bytes bytes); returns without synchronising."""
    ids = np.ascontiguousarray(request_ids, dtype=np.int64)
    _check(lib().gr_beams_get_batch_async(eng, ids.ctypes.data_as(C.POINTER(C.c_int64)), ids.shape[0],
                                          out_host, stream))


def gr_beams_result_bytes(eng: int) -> int:
    return int(lib().gr_beams_result_bytes(eng))


def gr_beams_unpack(eng: int, out_host: int, i: int, capacity: int, n_levels: int):
    """(codes [n][n_levels], scores [n]) of record i of a completed gr_beams_get_batch_async copy."""
    codes = np.zeros((max(capacity, 1), n_levels), dtype=np.int32)
    scores = np.zeros(max(capacity, 1), dtype=np.float32)
    nb = C.c_int32(0)
    _check(lib().gr_beams_unpack(eng, out_host, i, capacity, _host(codes), _host(scores), C.byref(nb)))
    return codes[: nb.value], scores[: nb.value]


def gr_score_items(eng: int, rid: int, items, stream: int = 0) -> np.ndarray:
    """Log-probability of each item ([n][n_levels] codes) over the request's context, in order."""
    it = np.ascontiguousarray(items, dtype=np.int32)
    scores = np.zeros(max(it.shape[0], 1), dtype=np.float32)
    _check(lib().gr_score_items(eng, rid, _host(it), it.shape[0], _host(scores), stream))
    return scores[: it.shape[0]]


def gr_score_items_batch(eng: int, request_ids, items, stream: int = 0) -> np.ndarray:
    """[n_requests][n] log-probabilities of items [n_requests][n][n_levels], one set of steps."""
    ids = np.ascontiguousarray(request_ids, dtype=np.int64)
    it = np.ascontiguousarray(items, dtype=np.int32)
    scores = np.zeros((ids.shape[0], it.shape[1]), dtype=np.float32)
    _check(lib().gr_score_items_batch(eng, ids.ctypes.data_as(C.POINTER(C.c_int64)), ids.shape[0], _host(it),
                                      it.shape[1], _host(scores), stream))
    return scores


def gr_score_items_labels(eng: int, request_ids, items, n_labels: int, stream: int = 0):
    """Item log-likelihoods [n_requests][n] and label log-probabilities [n_requests][n][n_labels]
    of items [n_requests][n][n_levels] (engines with a label head)."""
    ids = np.ascontiguousarray(request_ids, dtype=np.int64)
    it = np.ascontiguousarray(items, dtype=np.int32)
    scores = np.zeros((ids.shape[0], it.shape[1]), dtype=np.float32)
    labels = np.zeros((ids.shape[0], it.shape[1], n_labels), dtype=np.float32)
    _check(lib().gr_score_items_labels(eng, ids.ctypes.data_as(C.POINTER(C.c_int64)), ids.shape[0], _host(it),
                                       it.shape[1], _host(scores), _host(labels), stream))
    return scores, labels


def gr_request_release(eng: int, rid: int):
    _check(lib().gr_request_release(eng, rid))


def gr_request_reset(eng: int, rid: int, stream: int = 0):
    _check(lib().gr_request_reset(eng, rid, stream))


def gr_request_reset_batch(eng: int, request_ids, stream: int = 0):
    ids = np.ascontiguousarray(request_ids, dtype=np.int64)
    _check(lib().gr_request_reset_batch(eng, ids.ctypes.data_as(C.POINTER(C.c_int64)), ids.shape[0], stream))


def gr_last_error() -> str:
    return lib().gr_last_error().decode()


def gr_topk_select(cand, n_rows: int, V: int, k: int, out_flat, out_score, n_out, stream: int = 0):
    _check(lib().gr_topk_select(_ptr(cand), n_rows, V, k, _ptr(out_flat), _ptr(out_score), _ptr(n_out), stream))


def gr_debug_beam_state(eng: int, rid: int, capacity: int, n_levels: int, stream: int = 0):
    parent = np.zeros(capacity, dtype=np.int32)
    codes = np.zeros((capacity, n_levels), dtype=np.int32)
    scores = np.zeros(capacity, dtype=np.float32)
    n, level = C.c_int32(), C.c_int32()
    _check(lib().gr_debug_beam_state(eng, rid, capacity, _host(parent), _host(codes), _host(scores),
                                     C.byref(n), C.byref(level), stream))
    m = min(n.value, capacity)
    return {"n": n.value, "level": level.value, "parent": parent[:m], "codes": codes[:m, : level.value],
            "scores": scores[:m]}


def gr_debug_beam_path(eng: int, rid: int, capacity: int, n_levels: int, stream: int = 0):
    anc = np.zeros((capacity, n_levels), dtype=np.int32)
    n = C.c_int32()
    _check(lib().gr_debug_beam_path(eng, rid, capacity, _host(anc), C.byref(n), stream))
    return anc[: min(n.value, capacity)]


def gr_debug_chain_rows(eng: int, rid: int, layer: int, which: int, capacity: int, width: int, stream: int = 0):
    out = np.zeros((capacity, width), dtype=np.float32)
    n = C.c_int32()
    _check(lib().gr_debug_chain_rows(eng, rid, layer, which, capacity, _host(out), C.byref(n), stream))
    return out[: min(n.value, capacity)]


def gr_debug_hidden(eng: int, rid: int, capacity: int, hidden_dim: int, V: int, stream: int = 0):
    h = np.zeros((capacity, hidden_dim), dtype=np.float32)
    lg = np.zeros((capacity, V), dtype=np.float32)
    n = C.c_int32()
    _check(lib().gr_debug_hidden(eng, rid, capacity, _host(h), _host(lg), C.byref(n), stream))
    m = min(n.value, capacity)
    return h[:m], lg[:m]


def gr_debug_attn_out(eng: int, rid: int, layer: int, capacity: int, Hq: int, d: int, stream: int = 0):
    o = np.zeros((capacity, Hq, d), dtype=np.float32)
    n = C.c_int32()
    _check(lib().gr_debug_attn_out(eng, rid, layer, capacity, _host(o), C.byref(n), stream))
    return o[: min(n.value, capacity)]


def gr_engine_set_profiling(eng: int, enable: bool):
    _check(lib().gr_engine_set_profiling(eng, 1 if enable else 0))


def gr_engine_profile_read(eng: int, kind: int, level: int = -1):
    ms, n = C.c_double(), C.c_int64()
    _check(lib().gr_engine_profile_read(eng, kind, level, C.byref(ms), C.byref(n)))
    return ms.value, n.value


def gr_engine_profile_dispatches(eng: int, kind: int, level: int = -1) -> int:
    n = C.c_int64()
    _check(lib().gr_engine_profile_dispatches(eng, kind, level, C.byref(n)))
    return n.value


def gr_engine_set_profiling_kinds(eng: int, kinds: int):
    _check(lib().gr_engine_set_profiling_kinds(eng, kinds))


def gr_engine_set_profiling_stride(eng: int, stride: int):
    _check(lib().gr_engine_set_profiling_stride(eng, stride))


def gr_engine_graph_stats(eng: int):
    """(captures, replays) of a graph-replay engine."""
    a, b = C.c_int64(0), C.c_int64(0)
    _check(lib().gr_engine_graph_stats(eng, C.byref(a), C.byref(b)))
    return a.value, b.value


def gr_engine_profile_reset(eng: int):
    _check(lib().gr_engine_profile_reset(eng))


# ---------------------------------------------------------------- continuous-batching scheduler
def gr_sched_create(eng: int, max_active: int, stream: int = 0) -> int:
    out = C.c_void_p()
    _check(lib().gr_sched_create(eng, max_active, stream, C.byref(out)))
    return out.value


def gr_sched_destroy(sched: int):
    _check(lib().gr_sched_destroy(sched))


def gr_sched_submit(sched: int, rid: int, ctx_len: int, beam_width: int, k, v, q_last, flags: int = 0):
    _check(lib().gr_sched_submit(sched, rid, ctx_len, beam_width, _ptr(k), _ptr(v), _ptr(q_last), flags))


def gr_sched_advance(sched: int) -> int:
    n = C.c_int32()
    _check(lib().gr_sched_advance(sched, C.byref(n)))
    return n.value


def gr_sched_flush(sched: int) -> int:
    n = C.c_int32()
    _check(lib().gr_sched_flush(sched, C.byref(n)))
    return n.value


def gr_sched_completed(sched: int, capacity: int) -> np.ndarray:
    ids = np.zeros(max(capacity, 1), dtype=np.int64)
    n = C.c_int32()
    _check(lib().gr_sched_completed(sched, capacity, _host(ids), C.byref(n)))
    return ids[: min(n.value, capacity)]


def gr_sched_result(sched: int, rid: int, capacity: int, n_levels: int):
    codes = np.zeros((max(capacity, 1), n_levels), dtype=np.int32)
    scores = np.zeros(max(capacity, 1), dtype=np.float32)
    n = C.c_int32()
    _check(lib().gr_sched_result(sched, rid, capacity, _host(codes), _host(scores), C.byref(n)))
    return codes[: n.value], scores[: n.value]


def gr_sched_counts(sched: int):
    q, a, d, st = C.c_int32(), C.c_int32(), C.c_int32(), C.c_int64()
    _check(lib().gr_sched_counts(sched, C.byref(q), C.byref(a), C.byref(d), C.byref(st)))
    return {"queued": q.value, "active": a.value, "done": d.value, "steps": st.value}
