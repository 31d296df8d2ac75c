"""Pins of the prefill oracle (oracle/prefill.py) to facts other than its own code.

The soft token of the paper-daily article, section "Getting the user vector into the prompt:
three approaches", replaces a token's embedding by a projected user vector.  When the token
tables are built the way the stand-in reads them (a token's row at layer l = its embedding
times that layer's projection), a soft token whose embedding equals a token's embedding must
reproduce that token's rows exactly; a mistake in the projection's index order, the head
split or the layer index fails that."""
import numpy as np
import pytest

import oracle

L, VC, HQ, HKV, D, DE = 2, 7, 4, 2, 8, 16


def _embedded_tables(seed=0):
    rng = np.random.default_rng(seed)
    E = rng.standard_normal((VC, DE))
    wq = rng.standard_normal((L, DE, HQ * D))
    wk = rng.standard_normal((L, DE, HKV * D))
    wv = rng.standard_normal((L, DE, HKV * D))
    tq = np.einsum("ti,lic->ltc", E, wq).reshape(L, VC, HQ, D)
    tk = np.einsum("ti,lic->ltc", E, wk).reshape(L, VC, HKV, D)
    tv = np.einsum("ti,lic->ltc", E, wv).reshape(L, VC, HKV, D)
    return E, (wq, wk, wv), (tq, tk, tv)


@pytest.mark.parametrize("pos", [0, 3, 5])
def test_soft_token_with_a_tokens_embedding_equals_that_token(pos):
    E, (wq, wk, wv), (tq, tk, tv) = _embedded_tables()
    tokens = np.array([1, 4, 0, 6, 2, 5], dtype=np.int64)
    t_star = 3
    # identity projection: the user vector is the embedding itself
    K, V, q = oracle.prefill_context(tq, tk, tv, tokens, soft_pos=pos, user_vec=E[t_star], proj=np.eye(DE),
                                     w_q=wq, w_k=wk, w_v=wv)
    swapped = tokens.copy()
    swapped[pos] = t_star
    K0, V0, q0 = oracle.prefill_context(tq, tk, tv, swapped)
    np.testing.assert_allclose(K, K0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(V, V0, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(q, q0, rtol=1e-12, atol=1e-12)
    if pos == len(tokens) - 1:
        np.testing.assert_allclose(q, tq[:, t_star], rtol=1e-12, atol=1e-12)


def test_soft_token_at_the_last_position_gives_q_last():
    E, (wq, wk, wv), (tq, tk, tv) = _embedded_tables(1)
    tokens = np.array([2, 2, 6], dtype=np.int64)
    # a projection that maps a 3-dim user vector onto the embedding of token 4
    rng = np.random.default_rng(5)
    u = rng.standard_normal(3)
    proj = np.outer(u / (u @ u), E[4])
    _, _, q = oracle.prefill_context(tq, tk, tv, tokens, soft_pos=2, user_vec=u, proj=proj, w_q=wq, w_k=wk, w_v=wv)
    np.testing.assert_allclose(q, tq[:, 4], rtol=1e-10, atol=1e-10)


def test_soft_rows_are_linear_in_the_user_vector_and_zero_at_zero():
    _, (wq, wk, wv), (tq, tk, tv) = _embedded_tables(2)
    rng = np.random.default_rng(3)
    proj = rng.standard_normal((5, DE))
    u1, u2 = rng.standard_normal(5), rng.standard_normal(5)
    tokens = np.zeros(4, dtype=np.int64)

    def soft(u):
        K, V, _ = oracle.prefill_context(tq, tk, tv, tokens, soft_pos=1, user_vec=u, proj=proj, w_q=wq, w_k=wk,
                                         w_v=wv)
        return K[:, 1], V[:, 1]

    k1, v1 = soft(u1)
    k2, v2 = soft(u2)
    k12, v12 = soft(2.0 * u1 - 3.0 * u2)
    np.testing.assert_allclose(k12, 2.0 * k1 - 3.0 * k2, rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(v12, 2.0 * v1 - 3.0 * v2, rtol=1e-10, atol=1e-10)
    k0, v0 = soft(np.zeros(5))
    assert not k0.any() and not v0.any()


def test_token_positions_follow_the_token_order():
    _, _, (tq, tk, tv) = _embedded_tables(4)
    rng = np.random.default_rng(6)
    tokens = rng.integers(0, VC, 9)
    K, V, q = oracle.prefill_context(tq, tk, tv, tokens)
    perm = rng.permutation(9)
    Kp, Vp, _ = oracle.prefill_context(tq, tk, tv, tokens[perm])
    np.testing.assert_array_equal(Kp, K[:, perm])
    np.testing.assert_array_equal(Vp, V[:, perm])
    # two positions with the same token hold the same rows; the last token gives q_last
    same = [i for i in range(9) if tokens[i] == tokens[0]]
    for i in same:
        np.testing.assert_array_equal(K[:, i], K[:, 0])
    np.testing.assert_array_equal(q, tq[:, tokens[-1]])
    assert K.shape == (L, 9, HKV, D) and q.shape == (L, HQ, D)


def test_bf16_tables_decode_exactly():
    """Table rows given as bf16 bit patterns come out as their exact values."""
    bits = np.array([0x3F80, 0xC000, 0x3EAB, 0x0000], dtype=np.uint16)   # 1, -2, 0.333984375, 0
    t = np.broadcast_to(bits.reshape(1, 1, 1, 4), (1, 2, 1, 4)).copy()
    K, V, q = oracle.prefill_context(t, t, t, [1, 0])
    np.testing.assert_array_equal(K[0, :, 0], [[1.0, -2.0, 0.333984375, 0.0]] * 2)
