"""Plain float64 prefill of a request's context (oracle; test infrastructure only).

  [TRT-U] paper-daily.com, "Advancing Generative Recommendation Inference: our
          collaboration with NVIDIA on TensorRT LLM", section "Getting the user
          vector into the prompt: three approaches", third approach (soft token):
          the user's existing vector goes through one learned linear layer to a
          single token-sized embedding, which replaces a placeholder position of
          the prompt before the first forward pass.

Readings where the page is silent (the decode stand-in carries over):

* a context token's query, key and value at layer l are rows of per-layer
  tables indexed by its token id (as the fed-back code tables are for the
  decode step: no layer chain, so a position's K/V depend on that position
  only);
* the soft token has no table row; its embedding e = u @ proj is projected per
  layer with per-layer matrices, q = e @ w_q[l], k = e @ w_k[l],
  v = e @ w_v[l], head-major columns (head h, element i at h*d + i);
* the last position's query is the decode's first query (q_last).

Parity status: pinned in ``tests/test_oracle_prefill.py`` by the closed form
that a soft token whose embedding equals a token's embedding reproduces that
token's rows when the tables are built as embedding @ projection, by
linearity and zero in the user vector, and by a permuted-token check.
"""
from __future__ import annotations

import numpy as np

from .beam import as_f64


def soft_embedding(user_vec, proj) -> np.ndarray:
    """[TRT-U]: the one linear layer, user vector [du] -> embedding [de]."""
    return as_f64(user_vec) @ as_f64(proj)


def soft_qkv(e, w_q, w_k, w_v, n_q_heads: int, n_kv_heads: int, head_dim: int):
    """Per-layer q [L][Hq][d], k and v [L][Hkv][d] of a soft embedding e [de]."""
    e = np.asarray(e, dtype=np.float64)
    q = np.einsum("i,lic->lc", e, as_f64(w_q))
    k = np.einsum("i,lic->lc", e, as_f64(w_k))
    v = np.einsum("i,lic->lc", e, as_f64(w_v))
    L = q.shape[0]
    return (q.reshape(L, n_q_heads, head_dim), k.reshape(L, n_kv_heads, head_dim),
            v.reshape(L, n_kv_heads, head_dim))


def prefill_context(tok_q, tok_k, tok_v, tokens, soft_pos: int = -1, user_vec=None, proj=None, w_q=None,
                    w_k=None, w_v=None):
    """Context K, V [L][N][Hkv][d] and q_last [L][Hq][d], float64.

    tok_q [L][Vc][Hq][d], tok_k / tok_v [L][Vc][Hkv][d] (bf16 bit patterns or floats);
    position soft_pos (if >= 0) holds the soft token of user_vec instead of its token."""
    tq, tk, tv = as_f64(tok_q), as_f64(tok_k), as_f64(tok_v)
    tokens = np.asarray(tokens, dtype=np.int64)
    N = tokens.shape[0]
    L, _, Hkv, d = tk.shape
    Hq = tq.shape[2]
    K = np.zeros((L, N, Hkv, d))
    V = np.zeros((L, N, Hkv, d))
    soft = None
    if soft_pos >= 0:
        soft = soft_qkv(soft_embedding(user_vec, proj), w_q, w_k, w_v, Hq, Hkv, d)
    for n in range(N):
        if n == soft_pos:
            K[:, n] = soft[1]
            V[:, n] = soft[2]
        else:
            K[:, n] = tk[:, tokens[n]]
            V[:, n] = tv[:, tokens[n]]
    q_last = soft[0] if soft_pos == N - 1 else tq[:, tokens[N - 1]]
    return K, V, q_last
