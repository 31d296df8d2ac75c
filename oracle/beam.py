"""Plain float64 semantic-ID beam search (oracle; test infrastructure only).

Citations name the page and section; the pages print no formulas or code for
this path, so each function states the plain definition it implements.

  [BG]  paper-daily.com, "Advancing Generative Recommendation Inference: our
        collaboration with NVIDIA on TensorRT LLM", section "Background"
        (beam search keeps several highest-scoring prefixes, expands and
        prunes each step, the complete codes left are the candidates, and all
        of them are returned).
  [GR]  zhiding.cn article on NVIDIA recsys-examples, section
        "语义ID生成式推荐专用推理框架" (long shared context, short decode,
        wide beams, item-constrained generation / item-constrained top-K).
  [SID] same article, section "语义ID：解决稀疏性与长尾问题" (semantic IDs are
        decoded autoregressively and ranked by the output logits).
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, List, Sequence, Tuple

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) exactly: the 16 bits are the top half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def as_f64(x) -> np.ndarray:
    x = np.asarray(x)
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


# --------------------------------------------------------------------------- inputs
@dataclass
class Model:
    """Synthetic stand-in for the decoder, all float64.

    tq[l][t][c] : [Hq][d]   query at layer l of the token that feeds code c of level t back
    tk[l][t][c] : [Hkv][d]  its key,   tv[l][t][c] : [Hkv][d] its value
    w_sid[t]    : [Hq*d][V] projection of the hidden vector onto level t's codes
    """
    tq: np.ndarray
    tk: np.ndarray
    tv: np.ndarray
    w_sid: np.ndarray

    @property
    def n_layers(self): return self.tq.shape[0]
    @property
    def n_q_heads(self): return self.w_sid.shape[1] // self.head_dim
    @property
    def n_kv_heads(self): return self.tk.shape[3]
    @property
    def head_dim(self): return self.tq.shape[4]
    @property
    def n_levels(self): return self.w_sid.shape[0]
    @property
    def codebook(self): return self.w_sid.shape[2]

    @staticmethod
    def from_arrays(tq, tk, tv, w_sid) -> "Model":
        return Model(as_f64(tq), as_f64(tk), as_f64(tv), np.asarray(w_sid, dtype=np.float64))


@dataclass
class Request:
    """One request's shared context.

    ctx(l) -> (K [N][Hkv][d], V [N][Hkv][d]) float64 for layer l (may regenerate lazily)
    q_last : [L][Hq][d] query of the last context token (the query of decode step 0)
    """
    ctx: Callable[[int], Tuple[np.ndarray, np.ndarray]]
    q_last: np.ndarray


class PrefixSet:
    """The valid-prefix sets implied by an item list ([GR]: item-constrained generation).

    ``levels[t]`` holds every length-t prefix of an item as the integer
    sum_i c_i * V**(t-1-i) (big-endian), sorted.  The pages name no data
    structure; a sorted set per length is the plainest one."""

    def __init__(self, items: np.ndarray, V: int):
        items = np.asarray(items, dtype=np.int64)
        self.V = V
        self.n_levels = items.shape[1]
        self.levels = []
        for t in range(self.n_levels + 1):
            v = np.zeros(items.shape[0], dtype=np.int64)
            for i in range(t):
                v = v * V + items[:, i]
            self.levels.append(np.unique(v))

    def prefix_int(self, prefix: Sequence[int]) -> int:
        v = 0
        for c in prefix:
            v = v * self.V + int(c)
        return v

    def contains(self, prefix: Sequence[int]) -> bool:
        lv = self.levels[len(prefix)]
        x = self.prefix_int(prefix)
        i = np.searchsorted(lv, x)
        return bool(i < lv.shape[0] and lv[i] == x)

    def valid_codes(self, prefix: Sequence[int]) -> np.ndarray:
        """Codes c (ascending) such that prefix + (c,) is a prefix of some item."""
        nxt = self.levels[len(prefix) + 1]
        base = self.prefix_int(prefix) * self.V
        lo = np.searchsorted(nxt, base)
        hi = np.searchsorted(nxt, base + self.V)
        return (nxt[lo:hi] - base).astype(np.int64)


# --------------------------------------------------------------------------- attention
def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Softmax attention of one query over a whole sequence (no tiling, two passes).

    q [d], K [n][d], V [n][d]:  z = K q / sqrt(d);  p = exp(z - max z) / sum;  out = p V."""
    d = q.shape[0]
    z = K @ q / np.sqrt(d)
    z = z - z.max()
    p = np.exp(z)
    p = p / p.sum()
    return p @ V


def beam_sequence(req: Request, model: Model, prefix: Sequence[int], l: int):
    """The full sequence one beam attends over at layer l, and its query ([GR]).

    The beam's own decoded tokens follow the shared context: for a beam with
    codes c_0..c_{s-1} the sequence is ctx ++ [token(l, t, c_t) for t < s] and
    the query is that of its latest token (step 0: the last context token's).
    Built from the beam's own code tuple, never from shared buffers."""
    Kc, Vc = req.ctx(l)
    s = len(prefix)
    if s == 0:
        q = req.q_last[l]
        return q, Kc, Vc
    q = model.tq[l][s - 1][prefix[s - 1]]
    own_k = np.stack([model.tk[l][t][prefix[t]] for t in range(s)])
    own_v = np.stack([model.tv[l][t][prefix[t]] for t in range(s)])
    return q, np.concatenate([Kc, own_k], axis=0), np.concatenate([Vc, own_v], axis=0)


def beam_layer_output(req: Request, model: Model, prefix: Sequence[int], l: int) -> np.ndarray:
    """Attention output [Hq][d] of one beam at layer l; query head hq reads kv head hq // g."""
    q, K, V = beam_sequence(req, model, prefix, l)
    Hq, Hkv = q.shape[0], K.shape[1]
    g = Hq // Hkv
    out = np.empty((Hq, q.shape[1]))
    for hq in range(Hq):
        kv = hq // g
        out[hq] = attend(q[hq], K[:, kv, :], V[:, kv, :])
    return out


def beam_hidden(req: Request, model: Model, prefix: Sequence[int]) -> np.ndarray:
    """Hidden vector of one beam: sum over layers of the attention outputs, head-major [Hq*d]
    (a model with its own hidden_of, the layer chain of chain.py, computes it itself)."""
    if hasattr(model, "hidden_of"):
        return model.hidden_of(req, prefix)
    h = np.zeros(model.n_q_heads * model.head_dim)
    for l in range(model.n_layers):
        h += beam_layer_output(req, model, prefix, l).reshape(-1)
    return h


def codebook_logits(model: Model, h: np.ndarray, level: int) -> np.ndarray:
    """Logits over level `level`'s V codes: h @ w_sid[level] ([SID]: ranking by output logits)."""
    return h @ model.w_sid[level]


def constrained_log_softmax(logits: np.ndarray, valid: np.ndarray, norm: str = "valid") -> np.ndarray:
    """Log-probabilities of the valid codes ([GR]: item-constrained generation).

    norm="valid" (R2): normalise over the valid codes only.
    norm="full"  (R1): normalise over all V codes, then keep the valid ones."""
    dom = logits[valid] if norm == "valid" else logits
    m = dom.max()
    lse = m + np.log(np.sum(np.exp(dom - m)))
    return logits[valid] - lse


# --------------------------------------------------------------------------- beam search
def step_candidates(req: Request, model: Model, prefixes: PrefixSet,
                    beams: List[Tuple[tuple, float]], norm: str = "valid"):
    """Expand every beam by every valid code ([BG], [GR]).

    beams: [(prefix tuple, cumulative log-prob)] in slot order.
    Returns (score, j, c) arrays: score = beam score + log p(c | prefix)."""
    sc, js, cs = [], [], []
    for j, (prefix, score) in enumerate(beams):
        valid = prefixes.valid_codes(prefix)
        if valid.shape[0] == 0:
            continue
        h = beam_hidden(req, model, prefix)
        logp = constrained_log_softmax(codebook_logits(model, h, len(prefix)), valid, norm)
        sc.append(score + logp)
        js.append(np.full(valid.shape[0], j, dtype=np.int64))
        cs.append(valid)
    if not sc:
        return np.empty(0), np.empty(0, np.int64), np.empty(0, np.int64)
    return np.concatenate(sc), np.concatenate(js), np.concatenate(cs)


def select_topk(scores: np.ndarray, j: np.ndarray, c: np.ndarray, W: int, V: int):
    """Exhaustive sort: score descending, then flat index j*V + c ascending; keep min(W, n).

    Returns the indices (into the candidate arrays) of the kept candidates, in rank order."""
    order = np.lexsort((j * V + c, -scores))
    return order[: min(W, scores.shape[0])]


def score_items(req: Request, model: Model, prefixes: PrefixSet, items, norm: str = "valid") -> np.ndarray:
    """Log-probability of each given item under the item-constrained decode: the candidates
    are given and the model ranks them (paper-daily article, section "Background"), here by
    its own outputs (zhiding.cn article, section "语义ID": ranking via output logits).

    For item (c_0 .. c_{T-1}): sum over t of log p(c_t | c_0 .. c_{t-1}), each term the
    constrained log-softmax at the item's own prefix, added in level order; -inf from the
    first level whose code is not a valid child (the tuple is not an item)."""
    items = np.asarray(items, dtype=np.int64)
    out = np.empty(items.shape[0])
    memo = {}
    for i in range(items.shape[0]):
        total = 0.0
        for t in range(items.shape[1]):
            prefix = tuple(int(c) for c in items[i, :t])
            if prefix not in memo:
                valid = prefixes.valid_codes(prefix)
                if valid.shape[0] == 0:
                    memo[prefix] = {}
                else:
                    h = beam_hidden(req, model, prefix)
                    lp = constrained_log_softmax(codebook_logits(model, h, t), valid, norm)
                    memo[prefix] = dict(zip(valid.tolist(), lp.tolist()))
            lp_t = memo[prefix].get(int(items[i, t]))
            if lp_t is None:
                total = -np.inf
                break
            total = total + lp_t
        out[i] = total
    return out


def label_scores(req: Request, model: Model, items, w_label: np.ndarray) -> np.ndarray:
    """Label-token log-probabilities of given candidates (paper-daily article, sections
    "Background" and "Scoring many candidates at once": the candidates go into the prompt, each
    sees only the shared prefix and itself, and the model's log-probabilities of label tokens
    such as "yes" and "no", read after each candidate, rank them).

    Each candidate (c_0 .. c_{T-1}) is its own sequence: the context followed by its T code
    tokens (the model's tables hold a token for every level, T = n_levels); h is the hidden
    vector of its last token, whose query reads the context and all T tokens (beam_hidden of the
    full tuple); z = h @ w_label ([Hq*d][n_labels]) and the result row is z - logsumexp(z).
    Returns [n][n_labels]."""
    items = np.asarray(items, dtype=np.int64)
    w_label = np.asarray(w_label, dtype=np.float64)
    out = np.empty((items.shape[0], w_label.shape[1]))
    for i in range(items.shape[0]):
        h = beam_hidden(req, model, tuple(int(c) for c in items[i]))
        z = h @ w_label
        m = z.max()
        out[i] = z - (m + np.log(np.sum(np.exp(z - m))))
    return out


def beam_search(req: Request, model: Model, prefixes: PrefixSet, W: int, norm: str = "valid"):
    """Full decode of one request: n_levels steps from the empty prefix ([BG]).

    Returns a list with one entry per step s: the beam set B_{s+1} as
    [(prefix tuple, score, parent slot in B_s)], in slot (= rank) order.
    The last entry is the multi-beam result ([BG]: return every beam)."""
    beams = [((), 0.0)]
    history = []
    for _ in range(model.n_levels):
        sc, js, cs = step_candidates(req, model, prefixes, beams, norm)
        keep = select_topk(sc, js, cs, W, model.codebook)
        nxt = [(beams[js[i]][0] + (int(cs[i]),), float(sc[i]), int(js[i])) for i in keep]
        history.append(nxt)
        beams = [(p, s) for p, s, _ in nxt]
    return history
