"""Host-only checks of the C ABI: the library loads, exports every declared
symbol, and validates arguments and builds the item trie without touching a GPU."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import semantic_id_beam_amd as sib
from semantic_id_beam_amd import _lib as G
from tests.oracle_inputs import dict_trie

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x1000  # never dereferenced on the host


def _declared():
    with open(os.path.join(ROOT, "include", "gr_beam.h")) as f:
        src = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gr_[a-z_0-9]+)\s*\(", src, re.M)))


def test_library_exports_every_declared_symbol():
    L = sib.lib()
    decl = _declared()
    assert len(decl) >= 17
    for name in decl:
        assert hasattr(L, name), name
    assert sorted(G.EXPORTS) == decl


def test_wave_timeline_build_exports_the_same_symbols():
    # the measurement build (context-attention wave timeline compiled in) keeps the whole ABI
    path = os.path.join(os.path.dirname(G.__file__), "libgr_beam_timed.so")
    if not os.path.exists(path):
        pytest.skip("libgr_beam_timed.so not built")
    T = C.CDLL(path)
    for name in _declared():
        assert hasattr(T, name), name


def test_product_library_records_no_wave_timeline():
    L = sib.lib()
    buf = np.zeros(1024 * 8 * 8, dtype=np.int64)
    assert L.gr_wave_times_read(buf.ctypes.data_as(C.POINTER(C.c_int64)), 5) == G.GR_E_INVALID_ARG
    assert L.gr_wave_times_select(-2, 0) == G.GR_E_INVALID_ARG
    # the product library compiles no recorder: refused before any device call
    assert L.gr_wave_times_read(buf.ctypes.data_as(C.POINTER(C.c_int64)), buf.size) == G.GR_E_UNSUPPORTED


def _desc(L=1, Hq=4, Hkv=2, d=64, lv=3, V=16, dtype=G.GR_DTYPE_F32, norm=G.GR_NORM_VALID):
    return G.gr_model_desc(L, Hq, Hkv, d, lv, V, dtype, norm, FAKE, FAKE, FAKE, FAKE)


def _opts(R=1, W=4, ctx=64, S=0, flags=0, lpl=0):
    return G.gr_engine_opts(R, W, ctx, S, flags, lpl)


def _items(V=16, lv=3, n=200, seed=0):
    rng = np.random.default_rng(seed)
    flat = rng.choice(V ** lv, n, replace=False)
    return np.stack(np.unravel_index(flat, (V,) * lv), axis=1).astype(np.int32)


def test_create_and_trie_counts_match_dict_trie():
    items = _items()
    eng = G.gr_engine_create(_desc(), items, _opts())
    t = dict_trie(items)
    for s in range(4):
        expect = len({tuple(x[:s]) for x in items.tolist()})
        assert G.gr_engine_trie_nodes(eng, s) == expect
    assert G.gr_engine_workspace_bytes(eng) > 0
    assert len(t[()]) == G.gr_engine_trie_nodes(eng, 1)
    G.gr_engine_destroy(eng)


def test_duplicate_items_are_merged():
    items = _items()
    eng = G.gr_engine_create(_desc(), np.concatenate([items, items[:50]]), _opts())
    assert G.gr_engine_trie_nodes(eng, 3) == 200
    G.gr_engine_destroy(eng)


def test_workspace_grows_with_slots_and_pool():
    items = _items()
    a = G.gr_engine_create(_desc(), items, _opts(R=1, ctx=64))
    b = G.gr_engine_create(_desc(), items, _opts(R=4, ctx=64))
    c = G.gr_engine_create(_desc(), items, _opts(R=1, ctx=6400))
    wa, wb, wc = (G.gr_engine_workspace_bytes(x) for x in (a, b, c))
    assert wb > wa and wc > wa
    # pool: 2 (K,V) * L * Hkv * d * 4 bytes per padded token
    assert wc - wa == pytest.approx((6400 - 64) * 2 * 1 * 2 * 64 * 4, abs=1024)
    for x in (a, b, c):
        G.gr_engine_destroy(x)


@pytest.mark.parametrize("bad", [
    dict(d=96), dict(Hq=3, Hkv=2), dict(lv=0), dict(lv=9), dict(V=1), dict(V=2000), dict(dtype=7), dict(norm=3),
    dict(Hq=18, Hkv=1),
])
def test_create_rejects_bad_model(bad):
    with pytest.raises(G.GrError) as ei:
        G.gr_engine_create(_desc(**bad), _items(), _opts())
    assert ei.value.status in (G.GR_E_INVALID_ARG, G.GR_E_UNSUPPORTED)
    assert G.gr_last_error()


@pytest.mark.parametrize("bad", [dict(R=0), dict(W=0), dict(W=2000), dict(ctx=-1), dict(S=100), dict(lpl=-1)])
def test_create_rejects_bad_opts(bad):
    with pytest.raises(G.GrError):
        G.gr_engine_create(_desc(), _items(), _opts(**bad))


def test_create_rejects_bad_items():
    it = _items()
    it[5, 1] = 16
    with pytest.raises(G.GrError) as ei:
        G.gr_engine_create(_desc(), it, _opts())
    assert "code" in str(ei.value)
    with pytest.raises(G.GrError):
        G.gr_engine_create(_desc(), np.zeros((0, 3), np.int32), _opts())


def test_codebook_overflow_is_unsupported():
    with pytest.raises(G.GrError) as ei:
        G.gr_engine_create(_desc(lv=8, V=1024), np.zeros((1, 8), np.int32), _opts())
    assert ei.value.status == G.GR_E_UNSUPPORTED


def test_calls_before_bind_are_bad_state():
    eng = G.gr_engine_create(_desc(), _items(), _opts())
    with pytest.raises(G.GrError) as ei:
        G.gr_ctx_kv_load(eng, 1, 10, 4, FAKE, FAKE, FAKE)
    assert ei.value.status == G.GR_E_BAD_STATE
    with pytest.raises(G.GrError) as ei:
        G.gr_beam_step(eng, [1])
    assert ei.value.status == G.GR_E_BAD_STATE
    with pytest.raises(G.GrError) as ei:
        G.gr_request_release(eng, 1)
    assert ei.value.status == G.GR_E_NOT_FOUND
    with pytest.raises(G.GrError) as ei:
        G.gr_beams_get_batch(eng, [1], 4, 3)
    assert ei.value.status == G.GR_E_BAD_STATE
    with pytest.raises(G.GrError):
        G.gr_engine_bind_workspace(eng, FAKE + 1, 1 << 40)       # misaligned
    with pytest.raises(G.GrError) as ei:
        G.gr_engine_bind_workspace(eng, FAKE, 16)                # too small
    assert ei.value.status == G.GR_E_OUT_OF_MEMORY
    G.gr_engine_destroy(eng)


def test_padded_len_and_topk_args():
    assert G.gr_ctx_padded_len(1) == 64 and G.gr_ctx_padded_len(64) == 64 and G.gr_ctx_padded_len(65) == 128
    assert G.gr_ctx_padded_len(0) == 0
    for args in [(0, 16, 4), (4, 16, 0), (4, 16, 2000), (1 << 14, 1 << 13, 4)]:
        with pytest.raises(G.GrError):
            G.gr_topk_select(FAKE, *args, FAKE, FAKE, FAKE)


def test_null_engine_is_rejected():
    L = sib.lib()
    assert L.gr_beam_step(None, None, 0, None) == G.GR_E_INVALID_ARG
    assert L.gr_beams_get_batch(None, None, 1, 4, None, None, None, None) == G.GR_E_INVALID_ARG
    assert L.gr_engine_profile_dispatches(None, 0, -1, None) == G.GR_E_INVALID_ARG
    assert L.gr_score_items(None, 0, None, 1, None, None) == G.GR_E_INVALID_ARG
    assert L.gr_score_items_batch(None, None, 1, None, 1, None, None) == G.GR_E_INVALID_ARG
    assert L.gr_engine_set_profiling_stride(None, 4) == G.GR_E_INVALID_ARG
    assert L.gr_engine_destroy(None) == G.GR_OK
    assert L.gr_engine_workspace_bytes(None) == 0


def test_profiling_stride_must_be_positive():
    eng = G.gr_engine_create(_desc(), _items(), _opts())
    G.gr_engine_set_profiling_stride(eng, 4)
    G.gr_engine_set_profiling_stride(eng, 1)
    for bad in (0, -3):
        with pytest.raises(G.GrError) as ei:
            G.gr_engine_set_profiling_stride(eng, bad)
        assert ei.value.status == G.GR_E_INVALID_ARG
    G.gr_engine_destroy(eng)


def test_scheduler_host_checks():
    """The scheduler needs a bound engine and a concurrency cap within max_requests; null
    handles and outputs are rejected without touching a GPU."""
    L = sib.lib()
    eng = G.gr_engine_create(_desc(), _items(), _opts(R=4))
    with pytest.raises(G.GrError) as ei:
        G.gr_sched_create(eng, 2)
    assert ei.value.status == G.GR_E_BAD_STATE
    G.gr_engine_destroy(eng)
    out = C.c_void_p()
    assert L.gr_sched_create(None, 1, None, C.byref(out)) == G.GR_E_INVALID_ARG
    n = C.c_int32()
    assert L.gr_sched_advance(None, C.byref(n)) == G.GR_E_INVALID_ARG
    assert L.gr_sched_flush(None, C.byref(n)) == G.GR_E_INVALID_ARG
    assert L.gr_sched_submit(None, 1, 10, 4, FAKE, FAKE, FAKE, 0) == G.GR_E_INVALID_ARG
    assert L.gr_sched_result(None, 1, 4, None, None, C.byref(n)) == G.GR_E_INVALID_ARG
    assert L.gr_sched_completed(None, 0, None, C.byref(n)) == G.GR_E_INVALID_ARG
    assert L.gr_sched_counts(None, None, None, None, None) == G.GR_E_INVALID_ARG
    assert L.gr_sched_destroy(None) == G.GR_OK


def test_result_records_unpack_and_async_checks():
    """gr_beams_unpack reads a record (beam count, then codes [W_max][n_levels], then scores
    [W_max]) from host memory without a GPU; it refuses a capacity below the beam count and a
    count that no gather writes; the asynchronous gather needs a bound engine."""
    L = sib.lib()
    W, lv = 4, 3
    eng = G.gr_engine_create(_desc(), _items(), _opts(R=2, W=W))
    rb = G.gr_beams_result_bytes(eng)
    assert rb >= 16 + W * lv * 4 + W * 4 and rb % 16 == 0
    assert L.gr_beams_result_bytes(None) == 0
    buf = np.zeros(2 * rb, dtype=np.uint8)
    codes = np.arange(W * lv, dtype=np.int32).reshape(W, lv) + 100
    scores = -np.arange(1, W + 1, dtype=np.float32)
    rec = buf[rb:]
    rec[:4] = np.array([3], dtype=np.int32).view(np.uint8)
    rec[16:16 + codes.nbytes] = codes.view(np.uint8).ravel()
    rec[16 + codes.nbytes:16 + codes.nbytes + scores.nbytes] = scores.view(np.uint8)
    c, s = G.gr_beams_unpack(eng, buf.ctypes.data, 1, W, lv)
    np.testing.assert_array_equal(c, codes[:3])
    np.testing.assert_array_equal(s, scores[:3])
    c, s = G.gr_beams_unpack(eng, buf.ctypes.data, 0, W, lv)
    assert c.shape == (0, lv) and s.shape == (0,)
    n = C.c_int32()
    assert L.gr_beams_unpack(eng, buf.ctypes.data, 1, 2, G._host(np.zeros((2, lv), np.int32)),
                             G._host(np.zeros(2, np.float32)), C.byref(n)) == G.GR_E_INVALID_ARG
    assert n.value == 3
    rec[:4] = np.array([W + 1], dtype=np.int32).view(np.uint8)
    with pytest.raises(G.GrError):
        G.gr_beams_unpack(eng, buf.ctypes.data, 1, 64, lv)
    assert L.gr_beams_unpack(None, buf.ctypes.data, 0, 0, None, None, C.byref(n)) == G.GR_E_INVALID_ARG
    with pytest.raises(G.GrError) as ei:
        G.gr_beams_get_batch_async(eng, [0], buf.ctypes.data)
    assert ei.value.status == G.GR_E_BAD_STATE
    G.gr_engine_destroy(eng)
    ids = np.zeros(1, np.int64)
    assert L.gr_beams_get_batch_async(None, ids.ctypes.data_as(C.POINTER(C.c_int64)), 1, buf.ctypes.data,
                                      None) == G.GR_E_INVALID_ARG


def _label_desc(n_labels=2, w=FAKE, chain=None):
    import ctypes as C
    lab = G.gr_label_desc(n_labels, w)
    d = _desc()
    d.label = C.pointer(lab)
    if chain is not None:
        d.chain = C.pointer(chain)
    return d, lab


def test_label_head_grows_beamkv_and_adds_its_output():
    """A label head adds one level to BeamKV (the last code's key and value) and the label output
    rows; the engine keeps its own copy of the description."""
    plain = G.gr_engine_create(_desc(), _items(), _opts(R=2, W=8))
    d, lab = _label_desc(n_labels=5)
    labelled = G.gr_engine_create(d, _items(), _opts(R=2, W=8))
    wp, wl = G.gr_engine_workspace_bytes(plain), G.gr_engine_workspace_bytes(labelled)
    # per slot: K and V of one more level, L * W * Hkv * d * 4 bytes each (f32 model)
    assert wl - wp >= 2 * (2 * 1 * 8 * 2 * 64 * 4) + 2 * 8 * 5 * 4
    G.gr_engine_destroy(plain)
    G.gr_engine_destroy(labelled)


@pytest.mark.parametrize("n_labels,w,status", [(0, FAKE, "GR_E_UNSUPPORTED"), (17, FAKE, "GR_E_UNSUPPORTED"),
                                               (2, None, "GR_E_INVALID_ARG")])
def test_label_head_limits(n_labels, w, status):
    d, lab = _label_desc(n_labels=n_labels, w=w)
    with pytest.raises(G.GrError, match=status):
        G.gr_engine_create(d, _items(), _opts())


def test_label_head_is_not_for_the_layer_chain():
    chain = G.gr_chain_desc(64, 1e-6, *([FAKE] * 11))
    d, lab = _label_desc(chain=chain)
    d.dtype = G.GR_DTYPE_BF16
    d.n_q_heads, d.n_kv_heads, d.head_dim = 2, 1, 128
    with pytest.raises(G.GrError, match="GR_E_UNSUPPORTED"):
        G.gr_engine_create(d, _items(), _opts())


def test_label_scoring_needs_a_bound_engine_with_a_label_head():
    eng = G.gr_engine_create(_desc(), _items(), _opts())
    with pytest.raises(G.GrError, match="GR_E_BAD_STATE"):
        G.gr_score_items_labels(eng, [1], np.zeros((1, 2, 3), np.int32), 2)
    G.gr_engine_destroy(eng)
    d, lab = _label_desc()
    eng = G.gr_engine_create(d, _items(), _opts())
    with pytest.raises(G.GrError, match="GR_E_BAD_STATE"):
        G.gr_score_items_labels(eng, [1], np.zeros((1, 2, 3), np.int32), 2)
    G.gr_engine_destroy(eng)
