"""Parity of the HIP path (through the C ABI) with the CPU oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_harness import (SCORE_TOL, TeacherForced, attn_tol, check_beam_path, gpu_beams, load_request,
                               make_engine, rel_err_rows, save_report)
from tests.oracle_inputs import model_for, prefixes_for, request_for

pytestmark = pytest.mark.gpu


def _decode_checked(cfg, r=0, norm="valid", debug_attn=True, max_splits=0, check_attn_every=1, adopt=False):
    """Full decode of request r, each step checked against the oracle (teacher-forced)."""
    eng = make_engine(cfg, max_requests=1, debug_attn=debug_attn, norm=norm, max_splits=max_splits)
    rid = load_request(eng, cfg, r, rid=7, adopt=adopt)
    tf = TeacherForced(cfg, r, norm)
    prev = [()]
    tol = attn_tol(cfg)
    attn_errs = []
    for s in range(cfg.n_levels):
        eng.step([rid])
        after = gpu_beams(eng, rid)
        if debug_attn and s % check_attn_every == 0:
            for l in range(cfg.n_layers):
                got = eng.attn_out(rid, l)
                assert got.shape[0] == len(prev)
                ref = np.stack([oracle.beam_layer_output(tf.req, tf.model, p, l) for p in prev])
                err = rel_err_rows(got, ref)
                attn_errs.append(err)
                assert err <= tol, f"step {s} layer {l}: attention rel err {err}"
            h, lg = eng.hidden(rid)
            href = np.stack([oracle.beam_hidden(tf.req, tf.model, p) for p in prev])
            assert rel_err_rows(h, href) <= tol * max(1, cfg.n_layers)
        tf.check_step(prev, after)
        prev = after[0]
    codes, scores = eng.beams(rid)
    assert [tuple(c) for c in codes.tolist()] == prev
    eng.close()
    save_report(cfg, tf.report, attn_err=max(attn_errs) if attn_errs else None)
    return tf.report, codes, scores


def test_tiny_f32_decode_matches_oracle():
    cfg = synth.get_config("tiny_f32")
    rep, codes, scores = _decode_checked(cfg)
    # free-running comparison: the oracle's own search gives the same final beams
    hist = oracle.beam_search(request_for(cfg, 0), model_for(cfg), prefixes_for(cfg), 4, "valid")
    assert [p for p, _, _ in hist[-1]] == [tuple(c) for c in codes.tolist()]
    np.testing.assert_allclose(scores, [s for _, s, _ in hist[-1]], atol=1e-5)
    assert all(x["exact_order"] for x in rep)


def test_tiny_f32_full_vocab_normalisation():
    cfg = synth.get_config("tiny_f32")
    _decode_checked(cfg, norm="full")


def test_tiny_f32_wide_beam_is_exhaustive():
    cfg = synth.get_config("tiny_f32", beam_width=256)
    rep, codes, scores = _decode_checked(cfg, debug_attn=False)
    assert codes.shape[0] == cfg.n_items


def test_ctx1k_bf16_decode_matches_oracle():
    cfg = synth.get_config("ctx1k_beam256")
    rep, codes, scores = _decode_checked(cfg)
    assert codes.shape[0] == 256
    print("ctx1k report", rep)


@pytest.mark.parametrize("N", [1, 63, 64, 65, 129, 700])
def test_ragged_context_lengths(N):
    cfg = synth.get_config("ctx1k_beam256", ctx_len=N, beam_width=8, n_items=20000)
    _decode_checked(cfg)


@pytest.mark.parametrize("W", [1, 3, 33, 64, 100])
def test_beam_widths(W):
    cfg = synth.get_config("ctx1k_beam256", ctx_len=300, beam_width=W, n_items=20000)
    _decode_checked(cfg)


@pytest.mark.parametrize("hq,hkv,d,W", [(8, 8, 128, 96), (16, 4, 128, 64), (16, 8, 64, 64), (32, 4, 64, 16)])
def test_head_geometries(hq, hkv, d, W):
    """Query-head groups of 1, 4 and 8 and head_dim 64 in bf16 (the other workloads all use 16
    query / 8 kv heads of 128): g*W rows per kv head decide the context kernel (96 and 256
    rows at d = 128 take the 4- and 8-wave kernels, d = 64 the narrow ones)."""
    cfg = synth.get_config("ctx1k_beam256", n_q_heads=hq, n_kv_heads=hkv, head_dim=d, n_layers=2, ctx_len=500,
                           beam_width=W, n_items=20000)
    _decode_checked(cfg)


def test_two_layers_bf16_split_invariance():
    cfg = synth.get_config("ctx1k_beam256", n_layers=2, ctx_len=1500, beam_width=32, n_items=20000)
    _, c1, s1 = _decode_checked(cfg, max_splits=1)
    _, c2, s2 = _decode_checked(cfg, max_splits=16)
    # each run is within SCORE_TOL of the oracle, so they differ by at most twice that
    np.testing.assert_allclose(s1, s2, atol=2 * SCORE_TOL)


def test_adopt_equals_copy_bit_identical():
    cfg = synth.get_config("ctx1k_beam256", ctx_len=500, beam_width=64, n_items=20000)
    _, c1, s1 = _decode_checked(cfg, debug_attn=False)
    _, c2, s2 = _decode_checked(cfg, debug_attn=False, adopt=True)
    assert np.array_equal(c1, c2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))


def test_layered_wide_steps_match_oracle():
    """Wide steps of several requests without split partials: 4 requests x 2 row blocks (200
    beams x 2 query heads per kv head; the second block partly empty) x 8 kv heads x 4 layers
    per launch fill the chip, each workgroup over the whole context of one layer, whose last tile
    is ragged; with at most four layers per launch, the second launch holds only layers 4 and 5
    (its other workgroups stand idle).  Two requests are checked teacher-forced, with every
    layer's attention output of every beam (written by the kernel's own finish) and the hidden
    vector (the sum of the layers' fp16 partials).  The same step with every layer in one launch
    (the automatic choice here) gives the same beams, scores and hidden vectors bit for bit."""
    cfg = synth.get_config("ctx1k_beam256", n_requests=4, n_layers=6, ctx_len=700, beam_width=200, n_items=50000)
    eng = make_engine(cfg, max_requests=cfg.n_requests, debug_attn=True, max_layers_per_launch=4)
    rids = [load_request(eng, cfg, r) for r in range(cfg.n_requests)]
    checked = {0: TeacherForced(cfg, 0), 3: TeacherForced(cfg, 3)}
    prev = {r: [()] for r in checked}
    tol = attn_tol(cfg)
    errs = []
    for s in range(cfg.n_levels):
        eng.step(rids)
        for r, tf in checked.items():
            after = gpu_beams(eng, r)
            for l in range(cfg.n_layers):
                got = eng.attn_out(r, l)
                assert got.shape[0] == len(prev[r])
                ref = np.stack([oracle.beam_layer_output(tf.req, tf.model, p, l) for p in prev[r]])
                errs.append(rel_err_rows(got, ref))
                assert errs[-1] <= tol, f"request {r} step {s} layer {l}: attention rel err {errs[-1]}"
            h, _ = eng.hidden(r)
            href = np.stack([oracle.beam_hidden(tf.req, tf.model, p) for p in prev[r]])
            assert rel_err_rows(h, href) <= tol * cfg.n_layers
            tf.check_step(prev[r], after)
            prev[r] = after[0]
    def final(e, r):
        st = e.state(r)
        return st["codes"].copy(), st["scores"].copy(), e.hidden(r)[0].copy()

    split = {r: final(eng, r) for r in rids}
    eng.close()
    one = make_engine(cfg, max_requests=cfg.n_requests)
    for r in range(cfg.n_requests):
        load_request(one, cfg, r)
    for s in range(cfg.n_levels):
        one.step(rids)
    for r in rids:
        assert all(np.array_equal(a, b) for a, b in zip(split[r], final(one, r))), r
    one.close()
    save_report(cfg, checked[0].report + checked[3].report, attn_err=max(errs))


def test_layered_stream_steps_match_oracle():
    """Steps without split partials on two kernels at once: twelve narrow requests (30 beams x
    2 query heads = 60 rows per kv head) on the two-wave stream kernel, 8 kv heads x 4 layer
    slots per launch (at most four layers per launch), and two wide ones (150 beams) on the
    wide kernel, each group's launches on its own stream.  Each workgroup covers the whole (ragged, 333-token) context of one
    layer and merges the beam's own tokens (up to four, from BeamKV through the ancestry) in
    its prologue; the second launch of each group holds layer 4 alone.  Three requests are
    checked teacher-forced at every level with every layer's attention output and the hidden
    vector; the dispatch count shows the path."""
    from semantic_id_beam_amd import _lib as G
    shapes = ((333, 30),) * 12 + ((333, 150),) * 2
    cfg = synth.get_config("ctx2k_beam30_r64", n_requests=14, n_layers=5, shapes=shapes, n_items=50000)
    eng = make_engine(cfg, max_requests=cfg.n_requests, debug_attn=True, max_layers_per_launch=4)
    rids = [load_request(eng, cfg, r) for r in range(cfg.n_requests)]
    checked = {1: TeacherForced(cfg, 1), 10: TeacherForced(cfg, 10), 13: TeacherForced(cfg, 13)}
    prev = {r: [()] for r in checked}
    tol = attn_tol(cfg)
    errs = []
    G.gr_engine_set_profiling(eng.eng, True)
    for s in range(cfg.n_levels):
        eng.step(rids)
        for r, tf in checked.items():
            after = gpu_beams(eng, r)
            for l in range(cfg.n_layers):
                got = eng.attn_out(r, l)
                assert got.shape[0] == len(prev[r])
                ref = np.stack([oracle.beam_layer_output(tf.req, tf.model, p, l) for p in prev[r]])
                errs.append(rel_err_rows(got, ref))
                assert errs[-1] <= tol, f"request {r} step {s} layer {l}: attention rel err {errs[-1]}"
            h, _ = eng.hidden(r)
            href = np.stack([oracle.beam_hidden(tf.req, tf.model, p) for p in prev[r]])
            assert rel_err_rows(h, href) <= tol * cfg.n_layers
            tf.check_step(prev[r], after)
            prev[r] = after[0]
    G.gr_engine_set_profiling(eng.eng, False)
    for s in range(1, cfg.n_levels):   # level 0: one first-level launch; then 2 + 2 launches of 4 layer slots
        assert G.gr_engine_profile_dispatches(eng.eng, G.GR_PROF_CTX_ATTN, s) == 4, s
    eng.close()
    save_report(cfg, checked[1].report + checked[10].report + checked[13].report, attn_err=max(errs))


def test_mixed_variant_steps_match_oracle():
    """Continuous batching over every context-attention variant at once: six requests whose
    (context, beam width) pick the one-wave and two-wave streaming kernels, the four-wave
    narrow kernel, and the wide kernel (short and long contexts); the second half is
    admitted one step later, so the middle steps mix levels and variants (five groups, each
    group's chain of layer launches on its own stream, the fifth sharing the first's).  Each
    request is checked teacher-forced after each of its steps, with every layer's attention
    output of every beam and the hidden vector."""
    shapes = ((700, 8), (1500, 30), (900, 50), (2000, 100), (4100, 66), (600, 200))
    cfg = synth.get_config("ragged_r128", n_requests=6, n_layers=3, shapes=shapes, n_items=60000, waves=2)
    eng = make_engine(cfg, max_requests=cfg.n_requests, debug_attn=True)
    rids = [load_request(eng, cfg, r) for r in range(cfg.n_requests)]
    tfs = {r: TeacherForced(cfg, r) for r in rids}
    prev = {r: [()] for r in rids}
    level = {r: 0 for r in rids}
    tol = attn_tol(cfg)
    errs, report = [], []
    admitted = [0, 2, 4]
    for k in range(cfg.n_levels + 1):
        if k == 1:
            admitted += [1, 3, 5]
        step = [r for r in admitted if level[r] < cfg.n_levels]
        eng.step(step)
        for r in step:
            after = gpu_beams(eng, r)
            tf = tfs[r]
            for l in range(cfg.n_layers):
                got = eng.attn_out(r, l)
                assert got.shape[0] == len(prev[r])
                ref = np.stack([oracle.beam_layer_output(tf.req, tf.model, p, l) for p in prev[r]])
                errs.append(rel_err_rows(got, ref))
                assert errs[-1] <= tol, f"request {r} level {level[r]} layer {l}: attention rel err {errs[-1]}"
            h, _ = eng.hidden(r)
            href = np.stack([oracle.beam_hidden(tf.req, tf.model, p) for p in prev[r]])
            assert rel_err_rows(h, href) <= tol * cfg.n_layers
            tf.check_step(prev[r], after)
            prev[r] = after[0]
            level[r] += 1
    for r in rids:
        codes, _ = eng.beams(r)
        assert [tuple(c) for c in codes.tolist()] == prev[r]
        report += tfs[r].report
    eng.close()
    save_report(cfg, report, attn_err=max(errs))


def test_full_context_steps_mixing_levels_match_oracle():
    """Continuous batching on the full-context path: three admission waves of eight requests,
    one wave per step, so the middle steps hold requests at levels 0, 1 and 2 together (and
    the first step, all at level 0, runs the fused first level).  Beams of up to 128 rows
    (level-0 beams, 5, 30 and 50 beams) run on the two-wave stream kernel in 64-row blocks, the
    200-beam ones on the wide kernel, each workgroup over a whole (ragged, down to one-token)
    context; the dispatch count shows one launch per kernel and step instead of one per layer.
    Four requests (a narrow, a level-0-at-the-time, a two-block and a wide one) are checked
    teacher-forced after each of their steps, with every layer's attention output of every
    beam and the hidden vector."""
    from semantic_id_beam_amd import _lib as G
    wave = ((300, 30), (129, 5), (700, 50), (64, 30), (1, 30), (257, 5), (450, 200), (333, 30))
    shapes = wave + tuple((n + 37, w) for n, w in wave) + tuple((max(1, n - 20), w) for n, w in wave)
    cfg = synth.get_config("ragged_r128", n_requests=len(shapes), n_layers=4, shapes=shapes, n_items=60000,
                           waves=3)
    eng = make_engine(cfg, max_requests=cfg.n_requests, debug_attn=True)
    rids = [load_request(eng, cfg, r) for r in range(cfg.n_requests)]
    checked = (1, 10, 18, 22)
    tfs = {r: TeacherForced(cfg, r) for r in checked}
    prev = {r: [()] for r in rids}
    sets = {r: [] for r in rids}
    level = {r: 0 for r in rids}
    tol = attn_tol(cfg)
    errs, report, admitted, mixed = [], [], [], 0
    G.gr_engine_set_profiling(eng.eng, True)
    for k in range(3 + cfg.n_levels - 1):
        if k < 3:
            admitted += list(range(8 * k, 8 * k + 8))
        step = [r for r in admitted if level[r] < cfg.n_levels]
        mixed += len({level[r] for r in step}) > 1
        eng.step(step)
        for r in step:
            if r in tfs:
                after = gpu_beams(eng, r)
                tf = tfs[r]
                for l in range(cfg.n_layers):
                    got = eng.attn_out(r, l)
                    assert got.shape[0] == len(prev[r])
                    ref = np.stack([oracle.beam_layer_output(tf.req, tf.model, p, l) for p in prev[r]])
                    errs.append(rel_err_rows(got, ref))
                    assert errs[-1] <= tol, f"request {r} level {level[r]} layer {l}: attention rel err {errs[-1]}"
                h, _ = eng.hidden(r)
                href = np.stack([oracle.beam_hidden(tf.req, tf.model, p) for p in prev[r]])
                assert rel_err_rows(h, href) <= tol * cfg.n_layers
                tf.check_step(prev[r], after)
                sets[r].append(after[0])
                check_beam_path(eng, r, sets[r])   # BeamPath closure in mixed-level steps
                prev[r] = after[0]
            level[r] += 1
    G.gr_engine_set_profiling(eng.eng, False)
    assert mixed == 3
    # mixed-level steps are profiled under level n_levels: two kernels, all four layers each
    assert G.gr_engine_profile_dispatches(eng.eng, G.GR_PROF_CTX_ATTN, cfg.n_levels) == 2 * mixed
    for r in checked:
        codes, _ = eng.beams(r)
        assert [tuple(c) for c in codes.tolist()] == prev[r]
        report += tfs[r].report
    eng.close()
    save_report(cfg, report, attn_err=max(errs))


def test_max_beam_width_1024():
    """The largest beam width the engine takes: at the last step 1024 beams x 2 query heads =
    8 row blocks per kv head on the full-context wide path (2 requests x 2 layers), and the
    selection over 1024 x 256 candidates takes the streaming select.  Two requests, checked
    teacher-forced with every layer's attention output."""
    cfg = synth.get_config("ctx1k_beam256", n_requests=2, n_layers=2, ctx_len=300, beam_width=1024,
                           n_items=200000)
    eng = make_engine(cfg, max_requests=cfg.n_requests, debug_attn=True)
    rids = [load_request(eng, cfg, r) for r in range(cfg.n_requests)]
    tfs = {r: TeacherForced(cfg, r) for r in rids}
    prev = {r: [()] for r in rids}
    sets = {r: [] for r in rids}
    tol = attn_tol(cfg)
    errs = []
    for s in range(cfg.n_levels):
        eng.step(rids)
        for r, tf in tfs.items():
            after = gpu_beams(eng, r)
            for l in range(cfg.n_layers):
                got = eng.attn_out(r, l)
                assert got.shape[0] == len(prev[r])
                ref = np.stack([oracle.beam_layer_output(tf.req, tf.model, p, l) for p in prev[r]])
                errs.append(rel_err_rows(got, ref))
                assert errs[-1] <= tol, f"request {r} step {s} layer {l}: attention rel err {errs[-1]}"
            tf.check_step(prev[r], after)
            sets[r].append(after[0])
            check_beam_path(eng, r, sets[r])   # BeamPath closure at 1024 beams
            prev[r] = after[0]
    assert max(len(p) for p in prev.values()) == 1024
    eng.close()
    save_report(cfg, tfs[0].report + tfs[1].report, attn_err=max(errs))


def _candidates(cfg, n, n_bad, seed):
    """n candidates: items of the set (with repeats), n_bad code tuples outside it, shuffled."""
    rng = np.random.default_rng(seed)
    items = synth.items(cfg)
    ps = prefixes_for(cfg)
    good = items[rng.integers(0, items.shape[0], size=n - n_bad)]
    bad = []
    while len(bad) < n_bad:
        t = rng.integers(0, cfg.codebook, size=cfg.n_levels)
        if not ps.contains(tuple(int(c) for c in t)):
            bad.append(t)
    cands = np.concatenate([good, np.array(bad, dtype=good.dtype).reshape(-1, cfg.n_levels)])
    return cands[rng.permutation(cands.shape[0])].astype(np.int32)


def test_score_items_matches_oracle():
    """Candidate scoring: 500 given items (repeats and 20 tuples outside the item set among
    them) over one request's context, against the oracle's item log-probabilities; then the
    request's own beam search, whose final beams scored as candidates give their beam scores."""
    cfg = synth.get_config("ctx1k_beam256", n_layers=2, ctx_len=700, beam_width=64, n_items=50000)
    eng = make_engine(cfg, max_requests=1, max_beam_width=512)
    rid = load_request(eng, cfg, 0)
    cands = _candidates(cfg, 500, 20, seed=3)
    got = eng.score_items(rid, cands)
    ref = oracle.score_items(request_for(cfg, 0), model_for(cfg), prefixes_for(cfg), cands, "valid")
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin) and fin.sum() == 480
    err = float(np.max(np.abs(got[fin] - ref[fin])))
    assert err <= SCORE_TOL, err
    codes, scores = eng.beams(rid)                       # the candidates, in the given order
    assert np.array_equal(codes, cands) and np.array_equal(scores.view(np.uint32), got.view(np.uint32))
    eng.reset(rid)                                       # back to beam search on the same context
    for _ in range(cfg.n_levels):
        eng.step([rid])
    bcodes, bscores = eng.beams(rid)
    again = eng.score_items(rid, bcodes)
    np.testing.assert_allclose(again, bscores, rtol=0, atol=2 * SCORE_TOL)
    eng.close()
    save_report(cfg, [], score_err=err)


def test_score_items_batch_matches_oracle_and_single_calls():
    """Four requests' candidates scored in the same steps (full-context wide path at 300 beams
    x 2 layers): two requests against the oracle, all four against one call each."""
    cfg = synth.get_config("ctx1k_beam256", n_requests=4, n_layers=2, ctx_len=700, beam_width=64, n_items=50000)
    eng = make_engine(cfg, max_requests=cfg.n_requests, max_beam_width=512)
    rids = [load_request(eng, cfg, r) for r in range(cfg.n_requests)]
    cands = np.stack([_candidates(cfg, 300, 10, seed=20 + r) for r in rids])
    got = eng.score_items_batch(rids, cands)
    assert got.shape == (4, 300)
    for r in (0, 3):
        ref = oracle.score_items(request_for(cfg, r), model_for(cfg), prefixes_for(cfg), cands[r], "valid")
        fin = np.isfinite(ref)
        assert np.array_equal(np.isfinite(got[r]), fin)
        assert float(np.max(np.abs(got[r][fin] - ref[fin]))) <= SCORE_TOL
    for r in rids:
        one = eng.score_items(r, cands[r])
        fin = np.isfinite(one)
        assert np.array_equal(np.isfinite(got[r]), fin)
        np.testing.assert_allclose(got[r][fin], one[fin], rtol=0, atol=2 * SCORE_TOL)
    eng.close()


def test_score_all_items_is_a_distribution():
    """Under R2 the item probabilities sum to one: every item of the tiny float32 model scored
    on the GPU in one call."""
    cfg = synth.get_config("tiny_f32")
    eng = make_engine(cfg, max_requests=1, max_beam_width=256)
    rid = load_request(eng, cfg, 0)
    ps = prefixes_for(cfg)
    items = np.array([np.unravel_index(int(x), (cfg.codebook,) * cfg.n_levels) for x in ps.levels[-1]],
                     dtype=np.int32)
    got = eng.score_items(rid, items)
    ref = oracle.score_items(request_for(cfg, 0), model_for(cfg), ps, items, "valid")
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-5)
    assert abs(float(np.exp(got.astype(np.float64)).sum()) - 1.0) < 1e-5
    eng.close()


def _bf16_times_pow2(bits: np.ndarray, k: int) -> np.ndarray:
    """bf16 bit patterns times 2^k (exact: only the exponent moves)."""
    f = (bits.astype(np.uint32) << 16).view(np.float32) * np.float32(2.0 ** k)
    out = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal((out.astype(np.uint32) << 16).view(np.float32), f)
    return out


def test_value_range_power_of_two_scaling():
    """Attention is linear in V and the logits are h @ w_sid, so scaling every value row (context
    and beam tokens) by 2^k and w_sid by 2^-k leaves the search unchanged; in floating point the
    scaling is exact and commutes with every rounding, so the decode is bit-identical.  2^17
    takes |v| past fp16's range and 2^-30 far below its normal range: the split partials must
    hold both (16-bit o/l carries a per-head power-of-two scale)."""
    import semantic_id_beam_amd as sib
    from tests.engine_inputs import request_tensors
    cfg = synth.get_config("ctx1k_beam256", n_layers=2, ctx_len=700, beam_width=128, n_items=50000)
    _decode_checked(cfg, debug_attn=False)                 # the unscaled search is the oracle's
    tq, tk, tv = synth.token_tables(cfg)
    w = synth.w_sid(cfg)
    N, W = synth.request_shapes(cfg)[0]
    runs = []
    for k in (0, 17, -30):
        eng = sib.BeamEngine(tok_q=tq, tok_k=tk, tok_v=_bf16_times_pow2(tv, k), w_sid=w * np.float32(2.0 ** -k),
                             items=synth.items(cfg), n_layers=cfg.n_layers, n_q_heads=cfg.n_q_heads,
                             n_kv_heads=cfg.n_kv_heads, head_dim=cfg.head_dim, dtype=cfg.dtype, max_requests=1,
                             max_beam_width=W, max_ctx_tokens=sib._lib.lib().gr_ctx_padded_len(N))
        kc, vc, q = request_tensors(cfg, 0)
        eng.load(3, kc, vc * (2.0 ** k), q, W)
        for _ in range(cfg.n_levels):
            eng.step([3])
        runs.append(eng.beams(3))
        eng.close()
    for c, sc in runs[1:]:
        assert np.array_equal(c, runs[0][0])
        assert np.array_equal(sc.view(np.uint32), runs[0][1].view(np.uint32))


def test_determinism_bit_identical():
    cfg = synth.get_config("ctx1k_beam256", ctx_len=777, beam_width=128, n_items=50000)
    eng = make_engine(cfg, max_requests=1)
    rid = load_request(eng, cfg, 0)
    runs = []
    for _ in range(2):
        eng.reset(rid)
        for _ in range(cfg.n_levels):
            eng.step([rid])
        runs.append(eng.beams(rid))
    assert np.array_equal(runs[0][0], runs[1][0])
    assert np.array_equal(runs[0][1].view(np.uint32), runs[1][1].view(np.uint32))


def test_beams_get_batch_equals_single_calls():
    """The batched result path returns, bit for bit, what one gr_beams_get per request does;
    a batched reset rewinds every request to its root beam."""
    import semantic_id_beam_amd._lib as G
    cfg = synth.get_config("ctx1k_beam256", ctx_len=300, beam_width=48, n_items=5000)
    eng = make_engine(cfg, max_requests=3, max_ctx_tokens=3 * 320)
    rids = [load_request(eng, cfg, 0, rid=10), load_request(eng, cfg, 0, rid=11), load_request(eng, cfg, 0, rid=12)]
    eng.reset(rids[2])
    with pytest.raises(G.GrError) as ei:                        # nothing decoded yet
        eng.beams_batch(rids)
    assert ei.value.status == G.GR_E_BAD_STATE
    for _ in range(cfg.n_levels):
        eng.step(rids)
    single = [eng.beams(r) for r in rids]
    batch = eng.beams_batch(rids[::-1])[::-1]
    for (c1, s1), (c2, s2) in zip(single, batch):
        assert c1.shape[0] == cfg.beam_width
        assert np.array_equal(c1, c2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    eng.reset_batch(rids)                                       # rewind all at once, decode again
    for _ in range(cfg.n_levels):
        eng.step(rids)
    again = eng.beams_batch(rids)
    for (c1, s1), (c2, s2) in zip(single, again):
        assert np.array_equal(c1, c2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
    with pytest.raises(G.GrError) as ei:                        # capacity below the beam count
        G.gr_beams_get_batch(eng.eng, rids, cfg.beam_width - 1, cfg.n_levels, eng.stream)
    assert ei.value.status == G.GR_E_INVALID_ARG
    with pytest.raises(G.GrError) as ei:
        G.gr_beams_get_batch(eng.eng, [10, 99], cfg.beam_width, cfg.n_levels, eng.stream)
    assert ei.value.status == G.GR_E_NOT_FOUND
    eng.close()


def test_beams_get_batch_async_equals_sync():
    """The asynchronous gather (two pinned buffers, waited on with events) returns, bit for bit,
    what the synchronising batch call does, across more requests than one gather launch covers,
    while the next decode of the same requests is already enqueued behind it."""
    cfg = synth.get_config("ctx1k_beam256", ctx_len=65, beam_width=16, n_items=5000, n_layers=2)
    R = 70
    eng = make_engine(cfg, max_requests=R, max_ctx_tokens=R * 64 * 2)
    rids = [load_request(eng, cfg, 0, rid=100 + i) for i in range(R)]
    for _ in range(cfg.n_levels):
        eng.step(rids)
    ref = eng.beams_batch(rids)
    assert ref[0][0].shape[0] == cfg.beam_width
    bufs = [eng.result_buffer(R) for _ in range(2)]
    done0 = eng.beams_batch_async(rids, bufs[0])
    sub = rids[::-3]
    eng.reset_batch(sub)                                  # enqueued behind the first gather
    for _ in range(cfg.n_levels):
        eng.step(sub)
    done1 = eng.beams_batch_async(sub, bufs[1])
    done0.synchronize()
    for i in range(R):
        c, s = eng.unpack(bufs[0], i)
        assert np.array_equal(c, ref[i][0]) and np.array_equal(s.view(np.uint32), ref[i][1].view(np.uint32)), i
    done1.synchronize()
    for j, r in enumerate(sub):
        c, s = eng.unpack(bufs[1], j)
        c0, s0 = ref[r - 100]
        assert np.array_equal(c, c0) and np.array_equal(s.view(np.uint32), s0.view(np.uint32)), r
    eng.close()


def test_topk_select_bit_exact_vs_lexsort():
    import torch
    import semantic_id_beam_amd as sib
    rng = np.random.default_rng(5)
    cases = [(1, 16, 4, "r"), (7, 33, 20, "r"), (256, 256, 256, "r"), (30, 256, 30, "r"), (3, 1000, 1024, "r"),
             (64, 5, 300, "r"), (300, 256, 100, "r"),         # > 65536 candidates: streaming select
             (40, 128, 50, "eq"), (256, 256, 256, "n"), (1, 1024, 1024, "n"),
             (16, 256, 64, "off")]                           # array not on a 16-byte boundary
    for n_rows, V, k, kind in cases:
        if kind == "eq":                                     # one value: every candidate ties
            x = np.full((n_rows, V), -1.5, dtype=np.float32)
        elif kind == "n":                                    # continuous scores
            x = (rng.standard_normal((n_rows, V)) - 8).astype(np.float32)
        else:                                                # rounded: many exact ties
            x = np.round(rng.standard_normal((n_rows, V)) * 2, 2).astype(np.float32)
        x[rng.random((n_rows, V)) < 0.3] = -np.inf
        x[0, 0] = 0.0
        x[-1, -1] = -0.0
        if kind == "off":
            buf = torch.zeros(n_rows * V + 1, dtype=torch.float32, device="cuda")
            buf[1:] = torch.from_numpy(x.reshape(-1)).cuda()
            cand = buf[1:]
        else:
            cand = torch.from_numpy(x).cuda()
        of = torch.empty(k, dtype=torch.int32, device="cuda")
        os_ = torch.empty(k, dtype=torch.float32, device="cuda")
        no = torch.zeros(1, dtype=torch.int32, device="cuda")
        sib._lib.gr_topk_select(cand, n_rows, V, k, of, os_, no, torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        flat = np.arange(n_rows * V)
        xs = x.reshape(-1)
        fin = np.isfinite(xs)
        order = flat[fin][np.lexsort((flat[fin], -xs[fin].astype(np.float64)))]
        kk = min(k, order.shape[0])
        assert int(no.item()) == kk
        assert of.cpu().numpy()[:kk].tolist() == order[:kk].tolist()
        exp = xs[order[:kk]] + np.float32(0.0)          # -0 is reported as +0
        assert np.array_equal(os_.cpu().numpy()[:kk].view(np.uint32), exp.view(np.uint32))
