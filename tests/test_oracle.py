"""Pins of the CPU oracle against things other than itself.

Closed forms, a hand-derived worked example (tests/golden/worked_example.json),
library cross-checks (torch scaled_dot_product_attention in float64 on the CPU,
scipy log_softmax), brute-force enumeration, the greedy special case and
invariants.  Each pin is chosen so that a plausible slip in the oracle -- a
wrong scale, a dropped own token, the wrong table level or code, a transposed
head layout, mean instead of sum over layers, the wrong normalisation domain,
a reversed tie-break -- fails at least one of them.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle.beam import Model, PrefixSet, Request
from tests.oracle_inputs import dict_trie, model_for, prefixes_for, request_for

HERE = os.path.dirname(os.path.abspath(__file__))
rng = np.random.default_rng(1234)


def _ev(x):
    if isinstance(x, str):
        return float(eval(x, {"log": math.log, "__builtins__": {}}))
    if isinstance(x, list):
        return [_ev(v) for v in x]
    return float(x)


# ----------------------------------------------------------------- attention: closed forms
def test_attend_zero_query_is_mean_of_values():
    K, V = rng.standard_normal((37, 16)), rng.standard_normal((37, 16))
    np.testing.assert_allclose(oracle.attend(np.zeros(16), K, V), V.mean(0), rtol=0, atol=1e-13)


def test_attend_equal_keys_is_mean_of_values():
    K = np.tile(rng.standard_normal(16), (23, 1))
    V = rng.standard_normal((23, 16))
    np.testing.assert_allclose(oracle.attend(rng.standard_normal(16), K, V), V.mean(0), atol=1e-13)


def test_attend_single_token_returns_its_value():
    V = rng.standard_normal((1, 8))
    np.testing.assert_allclose(oracle.attend(rng.standard_normal(8), rng.standard_normal((1, 8)), V), V[0], atol=0)


def test_attend_constant_value_column():
    K, V = rng.standard_normal((50, 8)), rng.standard_normal((50, 8))
    V[:, 0] = 1.0
    assert abs(oracle.attend(rng.standard_normal(8) * 3, K, V)[0] - 1.0) < 1e-14


def test_attend_two_token_closed_form_uses_inverse_sqrt_d():
    # d = 9: scores are (q.k)/3.  q.k1 = 3*log(4) -> weight of token 1 = 4/5.
    d = 9
    q = np.zeros(d); q[0] = 1.0
    K = np.zeros((2, d)); K[1, 0] = 3 * math.log(4)
    V = np.zeros((2, d)); V[0, 1] = 1.0; V[1, 2] = 1.0
    o = oracle.attend(q, K, V)
    assert abs(o[1] - 0.2) < 1e-15 and abs(o[2] - 0.8) < 1e-15


def test_attend_is_permutation_invariant():
    K, V = rng.standard_normal((40, 16)), rng.standard_normal((40, 16))
    q = rng.standard_normal(16)
    p = rng.permutation(40)
    np.testing.assert_allclose(oracle.attend(q, K, V), oracle.attend(q, K[p], V[p]), atol=1e-13)


# ----------------------------------------------------------------- attention: library check
def _tiny_model(L=2, Hq=4, Hkv=2, d=8, V=5, lv=3, scale=1.0):
    T = lv - 1
    return Model(rng.standard_normal((L, T, V, Hq, d)) * scale, rng.standard_normal((L, T, V, Hkv, d)),
                 rng.standard_normal((L, T, V, Hkv, d)), rng.standard_normal((lv, Hq * d, V)))


def _tiny_request(L=2, N=11, Hq=4, Hkv=2, d=8):
    K = rng.standard_normal((L, N, Hkv, d)); Vv = rng.standard_normal((L, N, Hkv, d))
    return Request(ctx=lambda l: (K[l], Vv[l]), q_last=rng.standard_normal((L, Hq, d))), K, Vv


@pytest.mark.parametrize("prefix", [(), (3,), (1, 4)])
def test_layer_output_matches_torch_sdpa_gqa(prefix):
    import torch
    import torch.nn.functional as F
    m = _tiny_model()
    req, K, Vv = _tiny_request()
    for l in range(2):
        # the full sequence, assembled here from the tables by hand
        ks = [K[l]] + [m.tk[l][t][prefix[t]][None] for t in range(len(prefix))]
        vs = [Vv[l]] + [m.tv[l][t][prefix[t]][None] for t in range(len(prefix))]
        q = req.q_last[l] if not prefix else m.tq[l][len(prefix) - 1][prefix[-1]]
        kk = torch.from_numpy(np.concatenate(ks)).permute(1, 0, 2)[None]   # [1,Hkv,n,d]
        vv = torch.from_numpy(np.concatenate(vs)).permute(1, 0, 2)[None]
        qq = torch.from_numpy(q)[None, :, None, :]                          # [1,Hq,1,d]
        ref = F.scaled_dot_product_attention(qq, kk, vv, enable_gqa=True)[0, :, 0, :].numpy()
        np.testing.assert_allclose(oracle.beam_layer_output(req, m, prefix, l), ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- own tokens, query source, layers, layout
def test_own_token_comes_from_its_level_and_code():
    """A huge matching key on the own token of level 1 / code 2 pulls all attention onto it."""
    L, Hq, Hkv, d, V, lv = 1, 2, 1, 4, 3, 3
    tq = np.zeros((L, 2, V, Hq, d)); tk = np.zeros((L, 2, V, Hkv, d)); tv = np.zeros((L, 2, V, Hkv, d))
    tq[0, 1, 2, :, 0] = 50.0                 # query of level-1 code 2
    tk[0, 1, 2, 0, 0] = 50.0                 # key of level-1 code 2 (the beam's own token)
    tk[0, 0, :, 0, 1] = 50.0                 # level-0 keys: orthogonal to the query
    tv[0, 1, 2, 0] = [7, 8, 9, 10]
    tv[0, 0, :, 0] = -1
    m = Model(tq, tk, tv, np.zeros((lv, Hq * d, V)))
    req = Request(ctx=lambda l: (np.zeros((5, Hkv, d)), np.ones((5, Hkv, d))), q_last=np.zeros((L, Hq, d)))
    out = oracle.beam_layer_output(req, m, (0, 2), 0)
    np.testing.assert_allclose(out, [[7, 8, 9, 10]] * 2, atol=1e-9)


def test_step_query_is_previous_level_token_query():
    """At step 1 the query is tq[l][0][c0]; zeroing it makes attention uniform."""
    m = _tiny_model(L=1)
    m.tq[0, 0, 3] = 0.0
    req, K, Vv = _tiny_request(L=1)
    out = oracle.beam_layer_output(req, m, (3,), 0)
    seq_v = np.concatenate([Vv[0], m.tv[0, 0, 3][None]])
    g = 2
    for hq in range(4):
        np.testing.assert_allclose(out[hq], seq_v[:, hq // g].mean(0), atol=1e-13)


def test_hidden_sums_layers_head_major():
    """q = 0 everywhere -> each layer gives mean(V_l) per head; h is their sum, head-major."""
    L, Hq, Hkv, d = 3, 4, 2, 8
    m = _tiny_model(L=L, scale=0.0)
    req, K, Vv = _tiny_request(L=L)
    req.q_last[:] = 0.0
    h = oracle.beam_hidden(req, m, ())
    expect = np.zeros((Hq, d))
    for l in range(L):
        for hq in range(Hq):
            expect[hq] += Vv[l][:, hq // 2].mean(0)
    np.testing.assert_allclose(h, expect.reshape(-1), atol=1e-13)
    # and logits read h with head hq in rows hq*d .. hq*d+d-1
    np.testing.assert_allclose(oracle.codebook_logits(m, h, 0),
                               sum(expect[hq] @ m.w_sid[0][hq * d:(hq + 1) * d] for hq in range(Hq)), atol=1e-12)


# ----------------------------------------------------------------- log-softmax
def test_constrained_log_softmax_valid_normalises_over_valid():
    from scipy.special import log_softmax
    x = rng.standard_normal(32) * 3
    valid = np.array([1, 5, 6, 20, 31])
    lp = oracle.constrained_log_softmax(x, valid, "valid")
    assert abs(np.exp(lp).sum() - 1.0) < 1e-12
    np.testing.assert_allclose(lp, log_softmax(x[valid]), atol=1e-13)


def test_constrained_log_softmax_full_is_model_probability():
    from scipy.special import log_softmax
    x = rng.standard_normal(32) * 3
    valid = np.array([0, 2, 30])
    lp = oracle.constrained_log_softmax(x, valid, "full")
    assert np.exp(lp).sum() < 1.0
    np.testing.assert_allclose(lp, log_softmax(x)[valid], atol=1e-13)


def test_single_valid_child_has_zero_logprob_under_r2():
    assert oracle.constrained_log_softmax(np.array([5.0, -2.0, 1.0]), np.array([1]), "valid")[0] == 0.0


# ----------------------------------------------------------------- selection
def test_select_topk_matches_python_sort_with_ties():
    V = 7
    sc = np.round(rng.standard_normal(60), 1)          # many exact ties
    j, c = np.divmod(rng.permutation(60 * 3)[:60], V)
    for W in (1, 5, 60, 100):
        got = oracle.select_topk(sc, j, c, W, V)
        ref = sorted(range(60), key=lambda i: (-sc[i], j[i] * V + c[i]))[:min(W, 60)]
        assert got.tolist() == ref


def test_select_topk_hand_ties():
    # equal scores: lower flat index first; -inf last
    sc = np.array([1.0, 2.0, 2.0, -np.inf, 2.0])
    j = np.array([0, 1, 0, 0, 1]); c = np.array([0, 1, 3, 1, 0])      # flat = 0, 5, 3, 1, 4
    assert oracle.select_topk(sc, j, c, 5, 4).tolist() == [2, 4, 1, 0, 3]


# ----------------------------------------------------------------- prefix sets
def test_prefix_set_matches_dict_trie():
    items = np.array(sorted({tuple(x) for x in rng.integers(0, 6, size=(150, 3)).tolist()}))
    ps = PrefixSet(items, 6)
    t = dict_trie(items)
    for s in range(3):
        for p in itertools.product(range(6), repeat=s):
            exp = sorted(t.get(p, set()))
            assert ps.valid_codes(p).tolist() == exp
            assert ps.contains(p) == (p in t)


# ----------------------------------------------------------------- worked example (golden)
def _worked():
    with open(os.path.join(HERE, "golden", "worked_example.json")) as f:
        g = json.load(f)
    d = g["shape"]["head_dim"]
    tq = np.zeros((1, 1, 2, 1, d)); tk = np.zeros_like(tq); tv = np.zeros_like(tq)
    tq[0, 0] = _ev(g["tq_level0"]); tk[0, 0] = _ev(g["tk_level0"]); tv[0, 0] = _ev(g["tv_level0"])
    m = Model(tq, tk, tv, np.array(_ev(g["w_sid"])))
    K = np.array(_ev(g["ctx_k"])); Vv = np.array(_ev(g["ctx_v"]))
    req = Request(ctx=lambda l: (K, Vv), q_last=np.array(_ev(g["q_last"]))[None])
    return g, m, req, PrefixSet(np.array(g["items"]), 2)


def test_worked_example_attention_outputs():
    g, m, req, ps = _worked()
    e = g["expected"]
    np.testing.assert_allclose(oracle.beam_layer_output(req, m, (), 0), _ev(e["step0_attn_out"]), atol=1e-14)
    for c in ("0", "1"):
        np.testing.assert_allclose(oracle.beam_layer_output(req, m, (int(c),), 0),
                                   _ev(e["step1_attn_out"][c]), atol=1e-14)


@pytest.mark.parametrize("norm,key", [("valid", "R2"), ("full", "R1")])
@pytest.mark.parametrize("W", [2, 3])
def test_worked_example_beam_search(norm, key, W):
    g, m, req, ps = _worked()
    hist = oracle.beam_search(req, m, ps, W, norm)
    b1 = g["expected"]["B1"]["W2"]
    assert [(list(p), pa) for p, _, pa in hist[0]] == [(p, pa) for p, _, pa in b1]
    np.testing.assert_allclose([s for _, s, _ in hist[0]], [_ev(s) for _, s, _ in b1], atol=1e-14)
    exp = g["expected"]["valid"][key][f"W{W}"]
    assert [(list(p), pa) for p, _, pa in hist[1]] == [(p, pa) for p, _, pa in exp]
    np.testing.assert_allclose([s for _, s, _ in hist[1]], [_ev(s) for _, s, _ in exp], atol=1e-14)


# ----------------------------------------------------------------- beam search: special cases
def _tiny_cfg_inputs():
    import synth
    cfg = synth.get_config("tiny_f32")
    return cfg, model_for(cfg), request_for(cfg, 0), prefixes_for(cfg)


def _full_logp(req, m, ps, item, norm):
    """Brute-force scorer: sum of per-level log-probs along one item, prefix by prefix."""
    tot = 0.0
    for s in range(len(item)):
        pre = tuple(item[:s])
        valid = ps.valid_codes(pre)
        lp = oracle.constrained_log_softmax(oracle.codebook_logits(m, oracle.beam_hidden(req, m, pre), s), valid, norm)
        tot += lp[np.searchsorted(valid, item[s])]
    return tot


@pytest.mark.parametrize("norm", ["valid", "full"])
def test_beam_width_1_is_greedy(norm):
    cfg, m, req, ps = _tiny_cfg_inputs()
    hist = oracle.beam_search(req, m, ps, 1, norm)
    pre, score = (), 0.0
    for s in range(cfg.n_levels):
        valid = ps.valid_codes(pre)
        lp = oracle.constrained_log_softmax(oracle.codebook_logits(m, oracle.beam_hidden(req, m, pre), s), valid, norm)
        best = int(np.argmax(lp))                 # first maximum = smallest code on ties
        pre, score = pre + (int(valid[best]),), score + lp[best]
        assert hist[s][0][0] == pre and abs(hist[s][0][1] - score) < 1e-12


@pytest.mark.parametrize("norm", ["valid", "full"])
def test_wide_beam_equals_brute_force_enumeration(norm):
    """W >= every level's prefix count: the search keeps everything, so its result is
    every valid item ranked by its full-sequence score."""
    cfg, m, req, ps = _tiny_cfg_inputs()
    items = [tuple(int(v) for v in np.unravel_index(x, (cfg.codebook,) * cfg.n_levels)) for x in ps.levels[-1]]
    hist = oracle.beam_search(req, m, ps, 256, norm)
    brute = {it: _full_logp(req, m, ps, it, norm) for it in items}
    final = hist[-1]
    assert len(final) == len(items) == cfg.n_items
    assert {p for p, _, _ in final} == set(items)
    for p, s, _ in final:
        assert abs(s - brute[p]) < 1e-11
    scores = [s for _, s, _ in final]
    assert all(a >= b for a, b in zip(scores, scores[1:]))


@pytest.mark.parametrize("W", [1, 4, 7])
def test_beam_invariants_tiny(W):
    cfg, m, req, ps = _tiny_cfg_inputs()
    hist = oracle.beam_search(req, m, ps, W, "valid")
    prev = [((), 0.0)]
    for s, beams in enumerate(hist):
        n_valid = sum(len(ps.valid_codes(p)) for p, _ in prev)
        assert len(beams) == min(W, n_valid)
        for p, sc, pa in beams:
            assert ps.contains(p) and len(p) == s + 1
            assert p[:-1] == prev[pa][0]
            assert sc <= prev[pa][1] + 1e-15          # log-probs are <= 0
        scores = [b[1] for b in beams]
        assert all(a >= b for a, b in zip(scores, scores[1:]))
        prev = [(p, sc) for p, sc, _ in beams]


# ----------------------------------------------------------------- candidate scoring
@pytest.mark.parametrize("norm,key", [("valid", "R2"), ("full", "R1")])
def test_worked_example_item_scores(norm, key):
    """The hand-derived example's three items score their closed-form log-probabilities
    (under R2: log 1/2, log 1/3, log 1/6), and a tuple outside the item set scores -inf."""
    g, m, req, ps = _worked()
    exp = {tuple(p): _ev(s) for p, s, _ in g["expected"]["valid"][key]["W3"]}
    items = [list(k) for k in exp] + [[1, 0]]
    got = oracle.score_items(req, m, ps, items, norm)
    np.testing.assert_allclose(got[:-1], list(exp.values()), rtol=0, atol=1e-14)
    assert got[-1] == -np.inf


def test_item_probabilities_sum_to_one_under_r2():
    """R2 normalises every level over the valid children, so the items' probabilities form a
    distribution over the item set; R1 spends mass on invalid codes and never scores higher."""
    cfg, m, req, ps = _tiny_cfg_inputs()
    items = [np.unravel_index(x, (cfg.codebook,) * cfg.n_levels) for x in ps.levels[-1]]
    r2 = oracle.score_items(req, m, ps, items, "valid")
    r1 = oracle.score_items(req, m, ps, items, "full")
    assert len(items) == cfg.n_items
    assert abs(np.exp(r2).sum() - 1.0) < 1e-12
    assert np.all(r1 <= r2 + 1e-15) and np.exp(r1).sum() <= 1.0 + 1e-12


@pytest.mark.parametrize("norm", ["valid", "full"])
def test_item_scores_equal_exhaustive_beam_scores(norm):
    """W >= every level's prefix count: the search keeps every item, and its cumulative score
    is the item's score (same terms, same order)."""
    cfg, m, req, ps = _tiny_cfg_inputs()
    final = oracle.beam_search(req, m, ps, 256, norm)[-1]
    got = oracle.score_items(req, m, ps, [p for p, _, _ in final], norm)
    assert np.array_equal(got, np.array([s for _, s, _ in final]))


def test_tuples_outside_the_item_set_score_minus_inf():
    cfg, m, req, ps = _tiny_cfg_inputs()
    V = cfg.codebook
    item = np.unravel_index(int(ps.levels[-1][0]), (V,) * cfg.n_levels)
    pre = tuple(int(c) for c in item[:-1])
    bad_last = next(c for c in range(V) if c not in set(ps.valid_codes(pre).tolist()))
    bad_first = next(c for c in range(V) if c not in set(ps.valid_codes(()).tolist())) \
        if len(ps.valid_codes(())) < V else None
    tuples = [list(pre) + [bad_last]]
    if bad_first is not None:
        tuples.append([bad_first] + [0] * (cfg.n_levels - 1))
    got = oracle.score_items(req, m, ps, tuples + [list(item)], "valid")
    assert np.all(got[:-1] == -np.inf) and np.isfinite(got[-1])
