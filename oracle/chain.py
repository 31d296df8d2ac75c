"""A real layer chain for the decode step: float64 oracle (test infrastructure only).

The pages run the semantic-ID decode on Qwen3-1.7B (paper-daily.com, "Advancing Generative
Recommendation Inference: our collaboration with NVIDIA on TensorRT LLM", section
"Performance"; zhiding.cn recsys-examples article, section "语义ID生成式推荐专用推理框架": context
1,000 / 5,000, beam 256, Qwen3-1.7B).  They give no weights or arithmetic, so this module
defines a decoder of that shape with synthetic weights, in which layer l+1's new-token query,
key and value come from layer l's output (the table stand-in of ``beam.py`` has no such
dependency).  Readings where the pages are silent:

* a pre-norm decoder layer: RMSNorm, q/k/v projections (no bias), attention over the shared
  context plus the beam's own tokens (grouped-query, scale 1/sqrt(d), no positional rotation
  and no per-head norm, as in the table stand-in), output projection and residual; RMSNorm,
  SwiGLU MLP (down(silu(gate x) * up x)) and residual; a final RMSNorm gives the hidden vector
  that ``w_sid`` projects onto the level's codes;
* a fed-back code c of level t enters as the embedding row embed[t][c]; the first step's
  token is the last context token, whose input vector ``x_last`` the request supplies and
  whose key and value are already the context's last row (so it attends to the context only);
* the projections take bf16 inputs and accumulate in float32 on the GPU: the vectors that
  enter a projection (normed activations, the attention output, the SwiGLU product) and the
  projected q, k, v are rounded to bf16 (round to nearest even) at exactly those points, here
  and there; the residual stream, the norms and the hidden vector stay float (float64 here).

Each beam is recomputed as an independent full sequence (its tokens processed in order, each
attending to the context and to the beam's earlier tokens), nothing shared across beams.

Parity status: pinned by tests/test_oracle_chain.py (closed forms of the norm and of bf16
rounding, library cross-checks of RMSNorm, SiLU and bf16 rounding against torch, a torch
float64 re-implementation of the whole chain in matrix form with an attention mask, context
independence when the output projection is zero, an exact closed form of the hidden vector
when attention output and MLP are both zero, and brute-force enumeration through the generic
beam search).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence

import numpy as np

from .beam import Request, as_f64


def bf16_round(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    Two steps, each exact or a correct rounding: float64 -> float32 is round-to-nearest-even
    at 24 bits, and only values whose float32 image sits exactly half way between two bf16
    values could round differently from a direct 8-bit rounding; those are decided on the
    float64 value (double rounding guard)."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(invalid="ignore", over="ignore"):
        f = x.astype(np.float32)
        b = f.view(np.uint32).astype(np.uint64)
        low = b & 0xFFFF
        keep = b >> 16
        # candidate below (truncate) and above (next bf16 up in magnitude)
        lo = (keep << 16).astype(np.uint32).view(np.float32).astype(np.float64)
        hi = ((keep + 1) << 16).astype(np.uint32).view(np.float32).astype(np.float64)
        dlo, dhi = np.abs(x - lo), np.abs(hi - x)
        up = (dhi < dlo) | ((dhi == dlo) & ((keep & 1) == 1))
        out = np.where(up, hi, lo)
        out = np.where(low == 0, f.astype(np.float64), out)           # already a bf16 value
    return np.where(np.isfinite(x), out, x)


def rms_norm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps) * g


def silu(x: np.ndarray) -> np.ndarray:
    """x * sigmoid(x) = x / (1 + exp(-x))."""
    return x / (1.0 + np.exp(-x))


@dataclass
class ChainModel:
    """Weights (float64 copies of their bf16 / float32 values).

    embed   [levels-1][V][D]        input vector of a fed-back code of level t
    wq      [L][Hq*d][D]   wk, wv [L][Hkv*d][D]   (out x in)
    wo      [L][D][Hq*d]
    wg, wu  [L][I][D]      wd [L][D][I]
    g_attn, g_mlp [L][D]   g_final [D]  (RMSNorm gains)
    w_sid   [levels][D][V]
    """
    embed: np.ndarray
    wq: np.ndarray
    wk: np.ndarray
    wv: np.ndarray
    wo: np.ndarray
    wg: np.ndarray
    wu: np.ndarray
    wd: np.ndarray
    g_attn: np.ndarray
    g_mlp: np.ndarray
    g_final: np.ndarray
    w_sid: np.ndarray
    n_q_heads: int
    n_kv_heads: int
    eps: float = 1e-6

    @property
    def n_layers(self): return self.wq.shape[0]
    @property
    def head_dim(self): return self.wq.shape[1] // self.n_q_heads
    @property
    def hidden(self): return self.wq.shape[2]
    @property
    def n_levels(self): return self.w_sid.shape[0]
    @property
    def codebook(self): return self.w_sid.shape[2]

    def hidden_of(self, req, prefix) -> np.ndarray:
        return chain_hidden(req, self, prefix)

    @staticmethod
    def from_arrays(w: dict, w_sid, n_q_heads: int, n_kv_heads: int, eps: float = 1e-6) -> "ChainModel":
        f = {k: as_f64(w[k]) for k in ("embed", "wq", "wk", "wv", "wo", "wg", "wu", "wd", "g_attn", "g_mlp",
                                       "g_final")}
        return ChainModel(**f, w_sid=np.asarray(w_sid, dtype=np.float64), n_q_heads=n_q_heads,
                          n_kv_heads=n_kv_heads, eps=eps)


@dataclass
class ChainRequest:
    """One request of the chain model: its shared context (as ``beam.Request``) and the input
    vector of the last context token, [D]."""
    ctx: "callable"
    x_last: np.ndarray


def _attend_heads(q, K, V, g):
    """Per query head hq (kv head hq // g): softmax(q K^T / sqrt(d)) V, two passes, no tiling.
    q [Hq][d], K and V [n][Hkv][d] -> [Hq][d]."""
    d = q.shape[1]
    out = np.empty_like(q)
    for hq in range(q.shape[0]):
        z = K[:, hq // g, :] @ q[hq] / np.sqrt(d)
        p = np.exp(z - z.max())
        out[hq] = (p / p.sum()) @ V[:, hq // g, :]
    return out


def token_inputs(req: ChainRequest, model: ChainModel, prefix: Sequence[int]):
    """Input vectors of the tokens a beam runs through the layers: the last context token's for
    the empty prefix, else embed[t][c_t] for each fed-back code, in order."""
    if len(prefix) == 0:
        return [np.asarray(req.x_last, dtype=np.float64)], False
    return [model.embed[t][int(c)] for t, c in enumerate(prefix)], True


def beam_chain(req: ChainRequest, model: ChainModel, prefix: Sequence[int], record=None,
               rnd=bf16_round) -> np.ndarray:
    """Residual vectors after the last layer of every token of the beam's sequence, [T][D].

    The tokens go through the layers one after another; at layer l token t attends to the
    context's keys and values of layer l and to the keys and values (at layer l) of the beam's
    tokens 0..t (none for the first step's token, whose own row is in the context).  record, if
    given, receives per layer the attention outputs [T][Hq][d] (before rounding).  rnd is the
    rounding of a projection's input and of q, k, v (bf16; the identity gives the exact chain)."""
    xs, own = token_inputs(req, model, prefix)
    T, L = len(xs), model.n_layers
    Hq, Hkv, d = model.n_q_heads, model.n_kv_heads, model.head_dim
    g = Hq // Hkv
    x = [v.copy() for v in xs]
    for l in range(L):
        Kc, Vc = req.ctx(l)
        ks, vs, outs = [], [], []
        for t in range(T):
            xn = rnd(rms_norm(x[t], model.g_attn[l], model.eps))
            q = rnd(model.wq[l] @ xn).reshape(Hq, d)
            k = rnd(model.wk[l] @ xn).reshape(Hkv, d)
            v = rnd(model.wv[l] @ xn).reshape(Hkv, d)
            if own:
                ks.append(k)
                vs.append(v)
                K = np.concatenate([Kc, np.stack(ks)], axis=0)
                V = np.concatenate([Vc, np.stack(vs)], axis=0)
            else:
                K, V = Kc, Vc
            o = _attend_heads(q, K, V, g)
            outs.append(o)
            x[t] = x[t] + model.wo[l] @ rnd(o.reshape(-1))
            xm = rnd(rms_norm(x[t], model.g_mlp[l], model.eps))
            a = rnd(silu(model.wg[l] @ xm) * (model.wu[l] @ xm))
            x[t] = x[t] + model.wd[l] @ a
        if record is not None:
            record.append(np.stack(outs))
    return np.stack(x)


def chain_hidden(req: ChainRequest, model: ChainModel, prefix: Sequence[int]) -> np.ndarray:
    """The beam's hidden vector: the final RMSNorm of its last token's residual, [D]."""
    x = beam_chain(req, model, prefix)[-1]
    return rms_norm(x, model.g_final, model.eps)


def chain_layer_outputs(req: ChainRequest, model: ChainModel, prefix: Sequence[int]) -> np.ndarray:
    """Attention output of the beam's newest token at every layer, [L][Hq][d]."""
    rec = []
    beam_chain(req, model, prefix, record=rec)
    return np.stack([r[-1] for r in rec])
