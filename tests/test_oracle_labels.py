"""Pins of the oracle's label-token scoring (oracle.label_scores), on the CPU.

Each pin is fixed by something other than label_scores itself: the closed form of attention
with equal keys (the mean of the value rows), the one-label case, independence of a candidate
from the others in the list (each sees the context and itself only), and the equivalence with
the codebook path: reading the labels after a candidate is one more level of the item-scoring
decode whose projection is the label head, with every label valid."""
import numpy as np
import pytest

import oracle
import synth
from oracle.beam import Model, PrefixSet, Request
from oracle.inputs import label_model_for, request_for


def _log_softmax(z):
    m = z.max()
    return z - (m + np.log(np.sum(np.exp(z - m))))


def test_equal_keys_give_the_mean_of_every_value_row():
    rng = np.random.default_rng(5)
    L, Hq, Hkv, d, V, lv, N = 2, 4, 2, 8, 5, 3, 6
    key = rng.standard_normal(d)
    tq = rng.standard_normal((L, lv, V, Hq, d))
    tk = np.broadcast_to(key, (L, lv, V, Hkv, d)).copy()
    tv = rng.standard_normal((L, lv, V, Hkv, d))
    Kc = np.broadcast_to(key, (L, N, Hkv, d)).copy()
    Vc = rng.standard_normal((L, N, Hkv, d))
    model = Model(tq, tk, tv, rng.standard_normal((lv, Hq * d, V)))
    req = Request(ctx=lambda l: (Kc[l], Vc[l]), q_last=rng.standard_normal((L, Hq, d)))
    w_label = rng.standard_normal((Hq * d, 3))
    items = np.array([[0, 1, 2], [4, 4, 0], [3, 0, 1]])
    got = oracle.label_scores(req, model, items, w_label)
    g = Hq // Hkv
    for i, it in enumerate(items):
        h = np.zeros(Hq * d)
        for l in range(L):
            rows = np.concatenate([Vc[l], np.stack([tv[l, t, it[t]] for t in range(lv)])], axis=0)  # [N+lv][Hkv][d]
            mean = rows.mean(axis=0)
            h += np.concatenate([mean[hq // g] for hq in range(Hq)])
        np.testing.assert_allclose(got[i], _log_softmax(h @ w_label), rtol=1e-12, atol=1e-12)


def test_one_label_has_log_probability_zero():
    cfg = synth.get_config("tiny_f32")
    got = oracle.label_scores(request_for(cfg, 0), label_model_for(cfg), synth.items(cfg)[:7],
                              synth.w_label(cfg, 1))
    assert np.all(got == 0.0)


def test_a_candidate_does_not_see_the_other_candidates():
    cfg = synth.get_config("tiny_f32")
    req, model, w = request_for(cfg, 0), label_model_for(cfg), synth.w_label(cfg, 4)
    items = synth.items(cfg)[:9]
    full = oracle.label_scores(req, model, items, w)
    perm = np.random.default_rng(0).permutation(9)
    np.testing.assert_array_equal(oracle.label_scores(req, model, items[perm], w), full[perm])
    np.testing.assert_array_equal(oracle.label_scores(req, model, items[3:4], w), full[3:4])
    np.testing.assert_allclose(np.exp(full).sum(axis=1), 1.0, rtol=1e-12)


@pytest.mark.parametrize("norm", ["valid", "full"])
def test_labels_are_one_more_level_of_the_item_decode(norm):
    """With as many labels as codes, the label log-probabilities after an item equal the item
    decode's log-probabilities of one more level whose projection is the label head and whose
    codes are all valid after every item: score(item + (y,)) - score(item)."""
    cfg = synth.get_config("tiny_f32")
    req, model = request_for(cfg, 0), label_model_for(cfg)
    V = cfg.codebook
    w = synth.w_label(cfg, V)
    items = synth.items(cfg)[:12]
    ext = Model(model.tq, model.tk, model.tv, np.concatenate([model.w_sid, w[None].astype(np.float64)], axis=0))
    all_items = synth.items(cfg)
    ext_items = np.concatenate([np.repeat(all_items, V, axis=0), np.tile(np.arange(V), all_items.shape[0])[:, None]],
                               axis=1)
    ext_prefixes = PrefixSet(ext_items, V)
    prefixes = PrefixSet(all_items, V)
    got = oracle.label_scores(req, model, items, w)
    base = oracle.score_items(req, model, prefixes, items, norm)
    for y in range(V):
        q = np.concatenate([items, np.full((items.shape[0], 1), y)], axis=1)
        np.testing.assert_allclose(oracle.score_items(req, ext, ext_prefixes, q, norm) - base, got[:, y],
                                   rtol=1e-9, atol=1e-11)
