"""Pins of the layer-chain oracle (oracle/chain.py), on the CPU.

Each pin is fixed by something other than the oracle itself: closed forms of bf16 rounding
(ties to even, the double-rounding case), of RMSNorm and SiLU; torch's own bf16 conversion,
rms_norm and silu; a torch float64 re-implementation of the whole chain in matrix form (all of
a beam's tokens at once, causality through an attention mask, grouped-query attention through
scaled_dot_product_attention) against the oracle's token-by-token loop; context independence
and an exact closed form of the hidden vector when the attention output and the MLP are cut
off; brute-force enumeration through the generic beam search."""
import numpy as np
import pytest

import oracle
import synth
from oracle.chain import ChainModel, ChainRequest, beam_chain, bf16_round, chain_hidden, rms_norm, silu
from oracle.inputs import chain_model_for, chain_request_for, prefixes_for


def _cfg(**kw):
    base = dict(n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=384, ctx_len=40, beam_width=6,
                n_items=300, codebook=16)
    base.update(kw)
    return synth.get_config("chain_ctx5k_beam256_r8", **base)


# ---------------------------------------------------------------- bf16 rounding
def test_bf16_round_closed_forms():
    u = 2.0 ** -7                                  # bf16 spacing at 1 (7 stored fraction bits)
    cases = {
        1.0: 1.0,
        1.0 + u / 2: 1.0,                          # tie, 1.0 is even
        1.0 + 3 * u / 2: 1.0 + 2 * u,              # tie, 1 + u is odd
        1.0 + u / 2 + 2.0 ** -30: 1.0 + u,         # just above a tie: float32 would land on the tie
        -(1.0 + u / 2): -1.0,
        1.0 + 0.49 * u: 1.0,
        1.0 + 0.51 * u: 1.0 + u,
        0.0: 0.0,
        3.0 * 2.0 ** -133: 3.0 * 2.0 ** -133,      # a bf16 subnormal is kept
    }
    for x, want in cases.items():
        assert bf16_round(np.array([x]))[0] == want, x
    assert np.isnan(bf16_round(np.array([np.nan]))[0]) and bf16_round(np.array([np.inf]))[0] == np.inf


def test_bf16_round_matches_torch_on_float32_values():
    import torch
    rng = np.random.default_rng(3)
    x = (rng.standard_normal(200000) * np.exp(rng.uniform(-20, 20, 200000))).astype(np.float32)
    x[:1000] = (np.arange(1000, dtype=np.float32) + 0.5) * np.float32(2.0 ** -7) + 1.0   # ties
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(bf16_round(x.astype(np.float64)), want)


# ---------------------------------------------------------------- norm and activation
def test_rms_norm_closed_forms_and_torch():
    import torch
    g = np.array([1.0, 2.0, -0.5, 3.0])
    np.testing.assert_allclose(rms_norm(np.full(4, -7.0), g, 0.0), -g, rtol=1e-15)
    x = np.array([3.0, 4.0, 0.0, 0.0])              # mean square 25/4
    np.testing.assert_allclose(rms_norm(x, g, 0.0), x / 2.5 * g, rtol=1e-15)
    np.testing.assert_allclose(rms_norm(1e3 * x, g, 0.0), rms_norm(x, g, 0.0), rtol=1e-14)
    rng = np.random.default_rng(0)
    X, G = rng.standard_normal((5, 64)), rng.standard_normal(64)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(X), (64,), torch.from_numpy(G), eps=1e-6).numpy()
    np.testing.assert_allclose(rms_norm(X, G, 1e-6), ref, rtol=1e-13)


def test_silu_closed_forms_and_torch():
    import torch
    x = np.linspace(-30, 30, 1001)
    assert silu(np.array([0.0]))[0] == 0.0
    np.testing.assert_allclose(silu(x) - silu(-x), x, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(silu(np.array([50.0])), [50.0], rtol=1e-15)
    np.testing.assert_allclose(silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14)


# ---------------------------------------------------------------- the whole chain vs torch
def _torch_chain(req, m: ChainModel, prefix):
    """The chain in matrix form with torch float64: every token of the beam at once, causality
    from an attention mask over [context | own tokens], grouped-query attention by
    scaled_dot_product_attention (enable_gqa), no rounding.  Returns the final hidden vector and
    the newest token's attention output per layer."""
    import torch
    import torch.nn.functional as F
    T_ = torch.from_numpy
    L, Hq, Hkv, d = m.n_layers, m.n_q_heads, m.n_kv_heads, m.head_dim
    own = len(prefix) > 0
    X = T_(np.stack([m.embed[t][c] for t, c in enumerate(prefix)]) if own else np.asarray(req.x_last)[None])
    T = X.shape[0]
    outs = []
    for l in range(L):
        Kc, Vc = (T_(a) for a in req.ctx(l))
        N = Kc.shape[0]
        XN = F.rms_norm(X, (X.shape[1],), T_(m.g_attn[l]), eps=m.eps)
        Q = F.linear(XN, T_(m.wq[l])).view(T, Hq, d).transpose(0, 1)
        Ko = F.linear(XN, T_(m.wk[l])).view(T, Hkv, d)
        Vo = F.linear(XN, T_(m.wv[l])).view(T, Hkv, d)
        K = torch.cat([Kc, Ko], 0) if own else Kc
        V = torch.cat([Vc, Vo], 0) if own else Vc
        mask = torch.ones((T, K.shape[0]), dtype=torch.bool)
        if own:
            mask[:, N:] = torch.tril(torch.ones((T, T), dtype=torch.bool))
        O = F.scaled_dot_product_attention(Q[None], K.transpose(0, 1)[None].contiguous(),
                                           V.transpose(0, 1)[None].contiguous(), attn_mask=mask, enable_gqa=True)[0]
        O = O.transpose(0, 1)                                   # [T][Hq][d]
        outs.append(O[-1].numpy())
        X = X + F.linear(O.reshape(T, Hq * d), T_(m.wo[l]))
        XM = F.rms_norm(X, (X.shape[1],), T_(m.g_mlp[l]), eps=m.eps)
        X = X + F.linear(F.silu(F.linear(XM, T_(m.wg[l]))) * F.linear(XM, T_(m.wu[l])), T_(m.wd[l]))
    h = F.rms_norm(X[-1:], (X.shape[1],), T_(m.g_final), eps=m.eps)[0]
    return h.numpy(), np.stack(outs)


@pytest.mark.parametrize("prefix", [(), (5,), (5, 11), (0, 15)])
def test_chain_matches_torch_matrix_form(prefix):
    cfg = _cfg()
    m, req = chain_model_for(cfg), chain_request_for(cfg, 0)
    rec = []
    ident = lambda x: np.asarray(x, dtype=np.float64)
    x = beam_chain(req, m, prefix, record=rec, rnd=ident)
    h = rms_norm(x[-1], m.g_final, m.eps)
    h_ref, o_ref = _torch_chain(req, m, prefix)
    np.testing.assert_allclose(h, h_ref, rtol=1e-11, atol=1e-11)
    np.testing.assert_allclose(np.stack([r[-1] for r in rec]), o_ref, rtol=1e-11, atol=1e-12)
    # the rounded chain stays within the rounding's reach of the exact one, and differs from it
    hb = chain_hidden(req, m, prefix)
    assert 0 < np.max(np.abs(hb - h)) < 0.05 * np.max(np.abs(h))


def test_earlier_tokens_do_not_see_later_ones():
    cfg = _cfg()
    m, req = chain_model_for(cfg), chain_request_for(cfg, 1)
    x3 = beam_chain(req, m, (3, 7, 9)[:2])
    x2 = beam_chain(req, m, (3,))
    np.testing.assert_array_equal(x3[0], x2[0])


def _cut(m: ChainModel, wo=False, wd=False) -> ChainModel:
    import dataclasses
    kw = {}
    if wo:
        kw["wo"] = np.zeros_like(m.wo)
    if wd:
        kw["wd"] = np.zeros_like(m.wd)
    return dataclasses.replace(m, **kw)


def test_zero_output_projection_makes_the_context_irrelevant():
    cfg = _cfg()
    m = _cut(chain_model_for(cfg), wo=True)
    r0, r1 = chain_request_for(cfg, 0), chain_request_for(cfg, 1)
    r1_same_x = ChainRequest(ctx=r1.ctx, x_last=r0.x_last)
    for prefix in [(), (4,), (4, 2)]:
        np.testing.assert_array_equal(chain_hidden(r0, m, prefix), chain_hidden(r1_same_x, m, prefix))


def test_no_attention_output_no_mlp_closed_form():
    cfg = _cfg()
    m = _cut(chain_model_for(cfg), wo=True, wd=True)
    req = chain_request_for(cfg, 0)
    np.testing.assert_allclose(chain_hidden(req, m, ()), rms_norm(req.x_last, m.g_final, m.eps), rtol=1e-15)
    np.testing.assert_allclose(chain_hidden(req, m, (6, 13)), rms_norm(m.embed[1][13], m.g_final, m.eps), rtol=1e-15)


def test_chain_beam_search_exhaustive_equals_enumeration():
    cfg = _cfg(n_items=60, beam_width=60, codebook=8)
    m, req, ps = chain_model_for(cfg), chain_request_for(cfg, 0), prefixes_for(cfg)
    items = synth.items(cfg)
    hist = oracle.beam_search(req, m, ps, 60, "valid")
    got = {p: s for p, s, _ in hist[-1]}
    scores = oracle.score_items(req, m, ps, items)
    assert len(got) == items.shape[0]
    for it, sc in zip(items.tolist(), scores):
        assert abs(got[tuple(it)] - sc) < 1e-12
    assert abs(np.exp(scores).sum() - 1.0) < 1e-12                     # valid-code normalisation
    for level in hist:
        s = np.array([x[1] for x in level])
        assert np.all(s[:-1] >= s[1:])
