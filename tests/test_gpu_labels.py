"""Candidate scoring by label tokens on the GPU against the oracle (gr_score_items_labels).

Each candidate's codes run as its own tokens after the shared context (it sees the context and
itself only); the last code's hidden vector gives the label log-probabilities through the label
head.  Checked: the label log-probabilities against oracle.label_scores (1e-5 absolute on the
float32 model, 1e-3 on bf16, the log-prob bound of the decode), the item log-likelihoods of the
same call against oracle.score_items, and agreement between a batched call and single calls, up
to the pages' 500 candidates per request."""
import numpy as np
import pytest

import oracle
import synth
from oracle.inputs import label_model_for
from tests.gpu_harness import SCORE_TOL, load_request, make_engine, save_report
from tests.oracle_inputs import model_for, prefixes_for, request_for

pytestmark = pytest.mark.gpu


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


def _check(cfg, eng, rids, cands, n_labels, tol, checked):
    scores, labels = eng.score_items_labels(rids, cands)
    assert scores.shape == cands.shape[:2] and labels.shape == cands.shape[:2] + (n_labels,)
    errs = []
    for r in checked:
        req = request_for(cfg, r)
        ref = oracle.label_scores(req, label_model_for(cfg), cands[r], synth.w_label(cfg, n_labels))
        err = float(np.max(np.abs(labels[r] - ref)))
        assert err <= tol, (r, err)
        ref_s = oracle.score_items(req, model_for(cfg), prefixes_for(cfg), cands[r], "valid")
        fin = np.isfinite(ref_s)
        assert np.array_equal(np.isfinite(scores[r]), fin)
        assert float(np.max(np.abs(scores[r][fin] - ref_s[fin]))) <= max(tol, SCORE_TOL)
        errs.append(err)
    np.testing.assert_allclose(np.exp(labels.astype(np.float64)).sum(axis=2), 1.0, rtol=1e-5)
    return scores, labels, max(errs)


def test_labels_tiny_f32():
    """The float32 model: 40 candidates (5 outside the item set), three labels."""
    cfg = synth.get_config("tiny_f32")
    eng = make_engine(cfg, max_requests=1, max_beam_width=64, n_labels=3)
    rid = load_request(eng, cfg, 0)
    cands = _candidates(cfg, 40, 5, seed=1)[None]
    _, _, err = _check(cfg, eng, [rid], cands, 3, 1e-5, [0])
    eng.close()
    save_report(cfg, [], label_err=err)


@pytest.mark.parametrize("per_layer", [True, False])
def test_labels_bf16_batch(per_layer):
    """bf16, four requests x 200 candidates (10 outside the item set) x 4 layers in one call,
    two labels: one launch per layer (split-K), or (without the flag) full-context launches of
    several layers; two requests against the oracle, every request against a call of its own."""
    cfg = synth.get_config("ctx1k_beam256", n_requests=4, n_layers=4, ctx_len=300, beam_width=64, n_items=50000)
    eng = make_engine(cfg, max_requests=cfg.n_requests, max_beam_width=256, per_layer=per_layer, n_labels=2)
    rids = [load_request(eng, cfg, r) for r in range(cfg.n_requests)]
    cands = np.stack([_candidates(cfg, 200, 10, seed=40 + r) for r in rids])
    scores, labels, err = _check(cfg, eng, rids, cands, 2, SCORE_TOL, [0, 3])
    for r in rids:
        s1, l1 = eng.score_items_labels([r], cands[r][None])
        np.testing.assert_allclose(l1[0], labels[r], rtol=0, atol=2 * SCORE_TOL)
    eng.close()
    save_report(cfg, [], label_err=err, per_layer=per_layer)


def test_labels_500_candidates():
    """The pages' scoring workload shape: 500 candidates (20 outside the item set) of one
    request in one call, bf16, four labels, one launch per layer; every candidate against the
    oracle."""
    cfg = synth.get_config("ctx1k_beam256", n_requests=1, n_layers=3, ctx_len=400, beam_width=64, n_items=50000)
    eng = make_engine(cfg, max_requests=1, max_beam_width=512, per_layer=True, n_labels=4)
    rid = load_request(eng, cfg, 0)
    cands = _candidates(cfg, 500, 20, seed=77)[None]
    _, _, err = _check(cfg, eng, [rid], cands, 4, SCORE_TOL, [0])
    eng.close()
    save_report(cfg, [], label_err=err, n_candidates=500)


def test_labels_need_a_label_head():
    cfg = synth.get_config("tiny_f32")
    eng = make_engine(cfg, max_requests=1, max_beam_width=64)
    rid = load_request(eng, cfg, 0)
    import semantic_id_beam_amd._lib as G
    with pytest.raises(G.GrError, match="GR_E_BAD_STATE"):
        G.gr_score_items_labels(eng.eng, [rid], _candidates(cfg, 4, 0, seed=2)[None], 2, eng.stream)
    eng.close()
