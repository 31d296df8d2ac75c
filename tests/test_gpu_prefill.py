"""Prefill (gr_ctx_prefill) on the GPU against the oracle's prefill_context.

Token rows are copies of table rows, so they must match bit for bit; the soft token's rows
are float32 sums rounded to the model dtype, checked against the float64 oracle within the
bound of that arithmetic: one rounding to bf16 (2^-8 relative, above the half-ulp 2^-9 of
round to nearest) plus float32 accumulation over at most max(user_dim, embed_dim) terms,
2^-16 of the sum of the terms' magnitudes.  Padding tokens must be zero."""
import numpy as np
import pytest

import oracle
import synth
from tests.engine_inputs import make_engine
from tests.gpu_harness import SCORE_TOL
from tests.oracle_inputs import model_for, prefixes_for

pytestmark = pytest.mark.gpu

VOCAB, DU, DE = 500, 24, 200


def _cfg(n=300, dtype="bf16"):
    if dtype == "f32":
        return synth.get_config("tiny_f32", ctx_len=n)
    return synth.get_config("ctx1k_beam256", n_layers=3, ctx_len=n, beam_width=32, n_items=5000)


def _inputs(cfg):
    tabs = synth.prefill_tables(cfg, VOCAB)
    soft = synth.soft_token_weights(cfg, DU, DE)
    return tabs, soft


def _engine(cfg, tabs, soft, max_requests=2, max_ctx_tokens=None):
    eng = make_engine(cfg, max_requests=max_requests,
                      max_ctx_tokens=max_ctx_tokens or max_requests * synth.request_shapes(cfg)[0][0] + 64 * 8)
    eng.set_prefill(*tabs, *soft)
    return eng


def _to_f64(t):
    import torch
    if t.dtype == torch.bfloat16:
        return synth.bf16_bits_to_f32(t.view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
    return t.cpu().numpy().astype(np.float64)


def _native(cfg, N, fill=1.0):
    import torch
    Np = (N + 63) // 64 * 64
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    return (torch.full((L, H, Np, d), fill, dtype=dt, device="cuda"),
            torch.full((L, H, d, Np), fill, dtype=dt, device="cuda"),
            torch.zeros((L, cfg.n_q_heads, d), dtype=dt, device="cuda"))


def _soft_bound(u, soft, cfg, part):
    """2^-16 * sum of term magnitudes of the soft row's columns, [L][H][d] for part q/k/v."""
    proj, wq, wk, wv = (np.asarray(x, dtype=np.float64) for x in soft)
    u = np.asarray(u, dtype=np.float64)
    e_mag = np.abs(u) @ np.abs(proj) + np.abs(u @ proj)
    w = {"q": wq, "k": wk, "v": wv}[part]
    S = np.einsum("i,lic->lc", e_mag, np.abs(w))
    H = cfg.n_q_heads if part == "q" else cfg.n_kv_heads
    return 2.0 ** -16 * S.reshape(cfg.n_layers, H, cfg.head_dim)


def _check_soft(got, want, bound, dtype):
    rel = 2.0 ** -8 if dtype == "bf16" else 0.0
    err = np.abs(got - want) - (rel * np.abs(want) + bound)
    assert np.all(err <= 0), float(err.max())


@pytest.mark.parametrize("N,soft_pos", [(300, 7), (300, -1), (300, 299), (64, 0), (1, 0), (1, -1), (130, 64)])
def test_prefill_matches_oracle(N, soft_pos):
    import torch
    cfg = _cfg(N)
    tabs, soft = _inputs(cfg)
    eng = _engine(cfg, tabs, soft)
    toks = synth.prefill_tokens(cfg, 0, VOCAB, N)
    u = synth.user_vector(cfg, 0, DU)
    kn, vn, qo = _native(cfg, N)
    eng.prefill(5, toks, 32, soft_pos=soft_pos, user_vec=torch.from_numpy(u).cuda() if soft_pos >= 0 else None,
                k_native=kn, vt_native=vn, q_last_out=qo)
    torch.cuda.synchronize()
    K, V, q = oracle.prefill_context(*tabs, toks, soft_pos, u, *soft)
    Kd = _to_f64(kn[:, :, :N, :].permute(0, 2, 1, 3).contiguous())
    Vd = _to_f64(vn[:, :, :, :N].permute(0, 3, 1, 2).contiguous())
    tok_pos = [n for n in range(N) if n != soft_pos]
    np.testing.assert_array_equal(Kd[:, tok_pos], K[:, tok_pos])
    np.testing.assert_array_equal(Vd[:, tok_pos], V[:, tok_pos])
    if soft_pos >= 0:
        _check_soft(Kd[:, soft_pos], K[:, soft_pos], _soft_bound(u, soft, cfg, "k"), cfg.dtype)
        _check_soft(Vd[:, soft_pos], V[:, soft_pos], _soft_bound(u, soft, cfg, "v"), cfg.dtype)
    assert not kn[:, :, N:, :].float().abs().sum().item() and not vn[:, :, :, N:].float().abs().sum().item()
    qd = _to_f64(qo)
    if soft_pos == N - 1:
        _check_soft(qd, q, _soft_bound(u, soft, cfg, "q"), cfg.dtype)
    else:
        np.testing.assert_array_equal(qd, q)
    eng.close()


def test_prefill_f32_model_soft_token_last():
    import torch
    cfg = _cfg(77, dtype="f32")
    N = synth.request_shapes(cfg)[0][0]
    tabs, soft = _inputs(cfg)
    eng = _engine(cfg, tabs, soft)
    toks = synth.prefill_tokens(cfg, 1, VOCAB, N)
    u = synth.user_vector(cfg, 1, DU)
    kn, vn, qo = _native(cfg, N)
    eng.prefill(3, toks, 4, soft_pos=N - 1, user_vec=torch.from_numpy(u).cuda(), k_native=kn, vt_native=vn,
                q_last_out=qo)
    torch.cuda.synchronize()
    K, V, q = oracle.prefill_context(*tabs, toks, N - 1, u, *soft)
    Kd = _to_f64(kn[:, :, :N, :].permute(0, 2, 1, 3).contiguous())
    Vd = _to_f64(vn[:, :, :, :N].permute(0, 3, 1, 2).contiguous())
    np.testing.assert_array_equal(Kd[:, :N - 1], K[:, :N - 1])
    np.testing.assert_array_equal(Vd[:, :N - 1], V[:, :N - 1])
    _check_soft(Kd[:, N - 1], K[:, N - 1], _soft_bound(u, soft, cfg, "k"), "f32")
    _check_soft(Vd[:, N - 1], V[:, N - 1], _soft_bound(u, soft, cfg, "v"), "f32")
    _check_soft(_to_f64(qo), q, _soft_bound(u, soft, cfg, "q"), "f32")
    eng.close()


def test_decode_after_prefill_equals_loaded_context_and_oracle():
    """A request prefilled into the pool, one prefilled into caller buffers and one loaded
    (gr_ctx_kv_load) from those buffers decode bit-identically in the same steps; a request
    prefilled without a soft token (so its context equals the oracle's bit for bit) returns
    beams whose scores are the oracle's item scores over the oracle's prefilled context."""
    import torch
    cfg = _cfg(300)
    N, W, lv = 300, 32, cfg.n_levels
    tabs, soft = _inputs(cfg)
    eng = _engine(cfg, tabs, soft, max_requests=4, max_ctx_tokens=4 * 320)
    toks = synth.prefill_tokens(cfg, 2, VOCAB, N)
    u = torch.from_numpy(synth.user_vector(cfg, 2, DU)).cuda()
    eng.prefill(1, toks, W, soft_pos=11, user_vec=u)
    kn, vn, qo = _native(cfg, N, fill=0.0)
    eng.prefill(2, toks, W, soft_pos=11, user_vec=u, k_native=kn, vt_native=vn, q_last_out=qo)
    k = kn[:, :, :N, :].permute(0, 2, 1, 3).contiguous()
    v = vn[:, :, :, :N].permute(0, 3, 1, 2).contiguous()
    eng.load(3, k, v, qo, W)
    eng.prefill(4, toks, W)
    rids = [1, 2, 3, 4]
    for _ in range(lv):
        eng.step(rids)
    res = eng.beams_batch(rids)
    for r in (1, 2):
        assert np.array_equal(res[r][0], res[2][0]) and np.array_equal(res[r][1].view(np.uint32),
                                                                         res[2][1].view(np.uint32)), r
    assert res[0][0].shape[0] == W
    K, V, q = oracle.prefill_context(*tabs, toks)
    req = oracle.Request(ctx=lambda l: (K[l], V[l]), q_last=q)
    codes, scores = res[3]
    ps = prefixes_for(cfg)
    assert np.all(scores[:-1] >= scores[1:])
    for it in codes:
        assert ps.contains(tuple(int(x) for x in it))
    want = oracle.score_items(req, model_for(cfg), ps, codes)
    assert float(np.max(np.abs(want - scores))) <= SCORE_TOL
    eng.close()


def test_prefill_argument_checks():
    import semantic_id_beam_amd as sib
    cfg = _cfg(300)
    tabs, soft = _inputs(cfg)
    eng = make_engine(cfg, max_requests=2)
    toks = synth.prefill_tokens(cfg, 0, VOCAB, 300)
    with pytest.raises(sib.GrError) as ei:                   # no tables yet
        eng.prefill(1, toks, 8)
    assert ei.value.status == sib._lib.GR_E_BAD_STATE
    eng.set_prefill(*tabs)                                    # tables only: no soft token
    with pytest.raises(sib.GrError) as ei:
        eng.prefill(1, toks, 8, soft_pos=3, user_vec=1)
    assert ei.value.status == sib._lib.GR_E_BAD_STATE
    bad = toks.copy()
    bad[17] = VOCAB
    for kw in (dict(tokens=bad), dict(soft_pos=300), dict(soft_pos=-2), dict(beam_width=0)):
        args = dict(tokens=toks, beam_width=8, soft_pos=-1)
        args.update(kw)
        with pytest.raises(sib.GrError) as ei:
            eng.prefill(1, **args)
        assert ei.value.status == sib._lib.GR_E_INVALID_ARG, kw
    kn, vn, _ = _native(cfg, 300)
    with pytest.raises(sib.GrError) as ei:                   # one native buffer without the other
        eng.prefill(1, toks, 8, k_native=kn)
    assert ei.value.status == sib._lib.GR_E_INVALID_ARG
    eng.prefill(1, toks, 8)
    with pytest.raises(sib.GrError):                          # id already loaded
        eng.prefill(1, toks, 8)
    with pytest.raises(sib.GrError) as ei:                   # the pool holds one 300-token context
        eng.prefill(2, toks, 8)
    assert ei.value.status == sib._lib.GR_E_OUT_OF_MEMORY
    eng.prefill(2, toks, 8, k_native=kn, vt_native=vn)       # caller buffers need no pool
    eng.release(1)
    eng.release(2)
    eng.prefill(3, toks, 8)                                   # the released space is reused
    eng.close()


def test_prefill_full_size_sampled():
    """The headline shapes in the launch configuration the bench times (28 layers, 16/8
    heads of 128, a 5000-token context, the soft token first, user vector 256 -> embedding
    2048; vocabulary 4,096 here to keep the host tables small): sampled positions against the
    oracle, which computes a position from its own token alone, so it is given the sampled
    tokens' table rows only."""
    import torch
    cfg = synth.get_config("ctx5k_beam256_r8")
    vocab, du, de = 4096, 256, 2048
    N = synth.request_shapes(cfg)[0][0]
    tabs = synth.prefill_tables(cfg, vocab)
    soft = synth.soft_token_weights(cfg, du, de)
    eng = make_engine(cfg, max_requests=1)
    eng.set_prefill(*tabs, *soft)
    toks = synth.prefill_tokens(cfg, 0, vocab)
    u = synth.user_vector(cfg, 0, du)
    kn, vn, qo = _native(cfg, N)
    eng.prefill(0, toks, 256, soft_pos=0, user_vec=torch.from_numpy(u).cuda(), k_native=kn, vt_native=vn,
                q_last_out=qo)
    torch.cuda.synchronize()
    rng = np.random.default_rng(0)
    pos = np.unique(np.concatenate([[0, 1, 63, 64, 2047, 2048, N - 1], rng.integers(1, N, 25)]))
    uniq, inv = np.unique(toks[pos[1:]], return_inverse=True)
    sub = [t[:, uniq] for t in tabs]
    # position 0 is the soft token; the rest are the sampled tokens, in order
    K, V, q = oracle.prefill_context(*sub, np.concatenate([[0], inv]), 0, u, *soft)
    Kd = _to_f64(kn[:, :, torch.from_numpy(pos).cuda(), :].permute(0, 2, 1, 3).contiguous())
    Vd = _to_f64(vn[:, :, :, torch.from_numpy(pos).cuda()].permute(0, 3, 1, 2).contiguous())
    np.testing.assert_array_equal(Kd[:, 1:], K[:, 1:])
    np.testing.assert_array_equal(Vd[:, 1:], V[:, 1:])
    _check_soft(Kd[:, 0], K[:, 0], _soft_bound(u, soft, cfg, "k"), "bf16")
    _check_soft(Vd[:, 0], V[:, 0], _soft_bound(u, soft, cfg, "v"), "bf16")
    np.testing.assert_array_equal(_to_f64(qo), q)      # the last position is a token
    Np = kn.shape[2]
    assert not kn[:, :, N:, :].float().abs().sum().item() and not vn[:, :, :, N:].float().abs().sum().item()
    assert Np == 5056
    eng.close()
