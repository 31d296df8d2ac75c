"""Seeded generators.  Every function is a pure function of (config, indices)."""
from __future__ import annotations

import numpy as np
from scipy.special import ndtri

from .configs import Config

# tensor ids that enter the Philox key
_T_CTX_K, _T_CTX_V, _T_QLAST, _T_TQ, _T_TK, _T_TV, _T_WSID, _T_ITEMS, _T_SHAPES = range(1, 10)


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern, round to nearest even."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    b = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return b.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def times_pow2(x: np.ndarray, k: int) -> np.ndarray:
    """x * 2^k exactly: bf16 bit patterns (uint16) or float32.  Raises if a value would leave
    the exponent range (the product would not be exact)."""
    if k == 0:
        return x
    if x.dtype == np.uint16:
        f = bf16_bits_to_f32(x) * np.float32(2.0 ** k)
        out = (f.view(np.uint32) >> 16).astype(np.uint16)
        if not np.array_equal(bf16_bits_to_f32(out), f):
            raise ValueError("power-of-two scaling is not exact in bf16")
        return out
    out = (x.astype(np.float32) * np.float32(2.0 ** k)).astype(np.float32)
    if not np.array_equal(out * np.float32(2.0 ** -k), x.astype(np.float32)):
        raise ValueError("power-of-two scaling is not exact in float32")
    return out


def _make_table() -> np.ndarray:
    u = (np.arange(65536, dtype=np.float64) + 0.5) / 65536.0
    return _f32_to_bf16_bits(ndtri(u).astype(np.float32))


#: bf16 bit patterns of the 65536 quantiles of N(0,1): a discretised normal.
BF16_NORMAL_TABLE = _make_table()


def _key(cfg: Config, tensor: int, a: int = 0, b: int = 0) -> int:
    return ((cfg.seed & 0xFFFF) << 112) | (cfg.cfg_id << 96) | (tensor << 64) | ((a & 0xFFFFFFFF) << 32) | (b & 0xFFFFFFFF)


def _philox(cfg: Config, tensor: int, a: int = 0, b: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.Philox(key=_key(cfg, tensor, a, b)))


def _bf16_normal(gen: np.random.Generator, shape) -> np.ndarray:
    n = int(np.prod(shape))
    idx = np.frombuffer(gen.bytes(2 * n), dtype=np.uint16)
    return BF16_NORMAL_TABLE[idx].reshape(shape)


# ---------------------------------------------------------------- tiny fp32 config
_TINY_CACHE: dict = {}


def _tiny_all(cfg: Config) -> dict:
    """The tiny fp32 config: one default_rng(seed) stream, fixed tensor order."""
    key = cfg
    if key in _TINY_CACHE:
        return _TINY_CACHE[key]
    rng = np.random.default_rng(cfg.seed)
    V, lv = cfg.codebook, cfg.n_levels
    flat = rng.choice(V ** lv, size=cfg.n_items, replace=False)
    out = {"items": _decompose(np.sort(flat), V, lv)}
    n = request_shapes(cfg)[0][0]
    L, Hq, Hkv, d = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    out["ctx_k"] = rng.standard_normal((L, n, Hkv, d)).astype(np.float32)
    out["ctx_v"] = rng.standard_normal((L, n, Hkv, d)).astype(np.float32)
    out["q_last"] = rng.standard_normal((L, Hq, d)).astype(np.float32)
    T = max(lv - 1, 0)
    out["tq"] = rng.standard_normal((L, T, V, Hq, d)).astype(np.float32)
    out["tk"] = rng.standard_normal((L, T, V, Hkv, d)).astype(np.float32)
    out["tv"] = rng.standard_normal((L, T, V, Hkv, d)).astype(np.float32)
    out["w_sid"] = (rng.standard_normal((lv, Hq * d, V)) * np.sqrt(1.0 / (Hq * d))).astype(np.float32)
    _TINY_CACHE[key] = out
    return out


def _decompose(flat: np.ndarray, V: int, levels: int) -> np.ndarray:
    out = np.empty((flat.shape[0], levels), dtype=np.int32)
    x = flat.astype(np.int64)
    for t in range(levels - 1, -1, -1):
        out[:, t] = x % V
        x //= V
    return out


# ---------------------------------------------------------------- public API
def request_shapes(cfg: Config):
    """[(ctx_len, beam_width)] per request."""
    R = cfg.n_requests
    if cfg.shapes:
        assert len(cfg.shapes) == R
        return [(int(a), int(b)) for a, b in cfg.shapes]
    if isinstance(cfg.ctx_len, int) and isinstance(cfg.beam_width, int):
        return [(cfg.ctx_len, cfg.beam_width)] * R
    g = _philox(cfg, _T_SHAPES)
    if isinstance(cfg.ctx_len, int):
        ns = np.full(R, cfg.ctx_len, dtype=np.int64)
    else:
        lo, hi = cfg.ctx_len
        ns = g.integers(lo, hi + 1, size=R)
    if isinstance(cfg.beam_width, int):
        ws = np.full(R, cfg.beam_width, dtype=np.int64)
    else:
        ch = np.asarray(cfg.beam_width, dtype=np.int64)
        ws = ch[g.integers(0, len(ch), size=R)]
    return [(int(a), int(b)) for a, b in zip(ns, ws)]


def ctx_kv_block(cfg: Config, r: int, l: int):
    """Context K and V of request r, layer l, caller layout [N][Hkv][d].

    bf16 configs return uint16 bit patterns, fp32 configs float32 arrays."""
    n = request_shapes(cfg)[r][0]
    shape = (n, cfg.n_kv_heads, cfg.head_dim)
    if cfg.dtype == "f32":
        t = _tiny_all(cfg)
        return times_pow2(t["ctx_k"][l], cfg.k_scale_log2), t["ctx_v"][l]
    return (times_pow2(_bf16_normal(_philox(cfg, _T_CTX_K, r, l), shape), cfg.k_scale_log2),
            _bf16_normal(_philox(cfg, _T_CTX_V, r, l), shape))


def q_last(cfg: Config, r: int):
    """Query of the last context token, [L][Hq][d] (stands in for the prefill's last query)."""
    if cfg.dtype == "f32":
        return times_pow2(_tiny_all(cfg)["q_last"], cfg.q_scale_log2)
    return times_pow2(_bf16_normal(_philox(cfg, _T_QLAST, r), (cfg.n_layers, cfg.n_q_heads, cfg.head_dim)),
                      cfg.q_scale_log2)


def token_tables(cfg: Config):
    """(TQ [L][lv-1][V][Hq][d], TK [L][lv-1][V][Hkv][d], TV same as TK).

    Row (l, t, c) is the query/key/value at layer l of the token that feeds
    code c of level t back into the model."""
    if cfg.dtype == "f32":
        t = _tiny_all(cfg)
        return times_pow2(t["tq"], cfg.q_scale_log2), times_pow2(t["tk"], cfg.own_k_scale_log2), t["tv"]
    L, T, V = cfg.n_layers, max(cfg.n_levels - 1, 0), cfg.codebook
    tq = np.empty((L, T, V, cfg.n_q_heads, cfg.head_dim), dtype=np.uint16)
    tk = np.empty((L, T, V, cfg.n_kv_heads, cfg.head_dim), dtype=np.uint16)
    tv = np.empty_like(tk)
    for l in range(L):
        tq[l] = _bf16_normal(_philox(cfg, _T_TQ, l), tq.shape[1:])
        tk[l] = _bf16_normal(_philox(cfg, _T_TK, l), tk.shape[1:])
        tv[l] = _bf16_normal(_philox(cfg, _T_TV, l), tv.shape[1:])
    return times_pow2(tq, cfg.q_scale_log2), times_pow2(tk, cfg.own_k_scale_log2), tv


_T_LB_Q, _T_LB_K, _T_LB_V, _T_LB_W = range(30, 34)


def label_token_tables(cfg: Config):
    """Tables of the last level's codes as tokens (the label read of candidate scoring):
    (TQ [L][V][Hq][d], TK [L][V][Hkv][d], TV same as TK), drawn like token_tables (bf16: a Philox
    stream per tensor and layer; f32: normals from a stream of their own)."""
    L, V, Hq, Hkv, d = cfg.n_layers, cfg.codebook, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    if cfg.dtype == "f32":
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, cfg.cfg_id, _T_LB_Q]))
        tq = rng.standard_normal((L, V, Hq, d)).astype(np.float32)
        tk = rng.standard_normal((L, V, Hkv, d)).astype(np.float32)
        tv = rng.standard_normal((L, V, Hkv, d)).astype(np.float32)
        return times_pow2(tq, cfg.q_scale_log2), times_pow2(tk, cfg.own_k_scale_log2), tv
    tq = np.empty((L, V, Hq, d), dtype=np.uint16)
    tk = np.empty((L, V, Hkv, d), dtype=np.uint16)
    tv = np.empty_like(tk)
    for l in range(L):
        tq[l] = _bf16_normal(_philox(cfg, _T_LB_Q, l), tq.shape[1:])
        tk[l] = _bf16_normal(_philox(cfg, _T_LB_K, l), tk.shape[1:])
        tv[l] = _bf16_normal(_philox(cfg, _T_LB_V, l), tv.shape[1:])
    return times_pow2(tq, cfg.q_scale_log2), times_pow2(tk, cfg.own_k_scale_log2), tv


def token_tables_with_labels(cfg: Config):
    """token_tables with the label level appended: [L][n_levels][V][H][d] each."""
    base, last = token_tables(cfg), label_token_tables(cfg)
    return tuple(np.concatenate([b, x[:, None]], axis=1) for b, x in zip(base, last))


def w_label(cfg: Config, n_labels: int) -> np.ndarray:
    """Label head [Hq*d][n_labels] float32, N(0, 1/(Hq*d)) (variance), like w_sid."""
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, cfg.cfg_id, _T_LB_W, n_labels]))
    H = cfg.n_q_heads * cfg.head_dim
    return (rng.standard_normal((H, n_labels)) * np.sqrt(1.0 / H)).astype(np.float32)


def w_sid(cfg: Config) -> np.ndarray:
    """Codebook projection [levels][Hq*d][V] float32, N(0, 1/(Hq*d)) (variance)."""
    if cfg.dtype == "f32":
        return _tiny_all(cfg)["w_sid"]
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, cfg.cfg_id, _T_WSID]))
    H = cfg.n_q_heads * cfg.head_dim
    return (rng.standard_normal((cfg.n_levels, H, cfg.codebook)) * np.sqrt(1.0 / H)).astype(np.float32)


def items(cfg: Config) -> np.ndarray:
    """Valid items, [n_items][levels] int32, distinct, big-endian codes."""
    V, lv, n = cfg.codebook, cfg.n_levels, cfg.n_items
    if cfg.dtype == "f32":
        return _tiny_all(cfg)["items"]
    if cfg.item_dist == "uniform":
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, cfg.cfg_id, _T_ITEMS]))
        flat = rng.choice(V ** lv, size=n, replace=False)
        return _decompose(np.sort(flat), V, lv)
    if cfg.item_dist == "zipf":
        rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, cfg.cfg_id, _T_ITEMS]))
        ranks = np.arange(1, V + 1, dtype=np.float64)
        p = ranks ** (-cfg.zipf_a)
        p /= p.sum()
        perms = np.stack([rng.permutation(V) for _ in range(lv)])
        seen = np.empty(0, dtype=np.int64)
        first = np.empty(0, dtype=np.int64)    # draw position of each distinct tuple
        drawn = 0
        while seen.shape[0] < n:
            m = max(n, 1 << 16)
            codes = np.stack([perms[t][rng.choice(V, size=m, p=p)] for t in range(lv)], axis=1)
            flat = np.zeros(m, dtype=np.int64)
            for t in range(lv):
                flat = flat * V + codes[:, t]
            allf = np.concatenate([seen, flat])
            pos = np.concatenate([first, drawn + np.arange(m, dtype=np.int64)])
            uniq, idx = np.unique(allf, return_index=True)
            order = np.argsort(pos[idx], kind="stable")
            seen, first = uniq[order], pos[idx][order]
            drawn += m
        keep = seen[:n]
        return _decompose(np.sort(keep), V, lv)
    raise ValueError(cfg.item_dist)


# ---------------------------------------------------------------- prefill inputs
_T_PF_TAB, _T_PF_TOK, _T_PF_USER, _T_PF_PROJ, _T_PF_W = range(10, 15)


def _normal(cfg: Config, gen: np.random.Generator, shape, scale: float = 1.0):
    """bf16 bit patterns of N(0, scale^2) for bf16 configs (scale 1 only), float32 otherwise."""
    if cfg.dtype == "bf16" and scale == 1.0:
        return _bf16_normal(gen, shape)
    return (gen.standard_normal(shape) * scale).astype(np.float32)


def prefill_tables(cfg: Config, vocab: int):
    """(TQ [L][Vc][Hq][d], TK [L][Vc][Hkv][d], TV same as TK): per-layer rows of the
    context tokens, N(0, 1) in the model dtype (bf16 bit patterns or float32)."""
    L, Hq, Hkv, d = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    return (_normal(cfg, _philox(cfg, _T_PF_TAB, 0), (L, vocab, Hq, d)),
            _normal(cfg, _philox(cfg, _T_PF_TAB, 1), (L, vocab, Hkv, d)),
            _normal(cfg, _philox(cfg, _T_PF_TAB, 2), (L, vocab, Hkv, d)))


def prefill_tokens(cfg: Config, r: int, vocab: int, n: int | None = None) -> np.ndarray:
    """Context token ids of request r, [N] int32, uniform over [0, vocab)."""
    if n is None:
        n = request_shapes(cfg)[r][0]
    return _philox(cfg, _T_PF_TOK, r).integers(0, vocab, n, dtype=np.int32)


def user_vector(cfg: Config, r: int, user_dim: int) -> np.ndarray:
    """User vector of request r, [user_dim] float32, N(0, 1)."""
    return _philox(cfg, _T_PF_USER, r).standard_normal(user_dim).astype(np.float32)


def soft_token_weights(cfg: Config, user_dim: int, embed_dim: int):
    """(proj [user_dim][embed_dim] with variance 1/user_dim, w_q [L][embed_dim][Hq*d], w_k and
    w_v [L][embed_dim][Hkv*d] with variance 1/embed_dim), float32: projected entries come out
    about N(0, 1) like the table rows."""
    L, Hq, Hkv, d = cfg.n_layers, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    g = lambda i, shape, var: (_philox(cfg, _T_PF_W, i).standard_normal(shape) * np.sqrt(var)).astype(np.float32)
    proj = (_philox(cfg, _T_PF_PROJ).standard_normal((user_dim, embed_dim)) * np.sqrt(1.0 / user_dim)).astype(np.float32)
    return (proj, g(0, (L, embed_dim, Hq * d), 1.0 / embed_dim), g(1, (L, embed_dim, Hkv * d), 1.0 / embed_dim),
            g(2, (L, embed_dim, Hkv * d), 1.0 / embed_dim))


# ---------------------------------------------------------------- layer-chain weights
_T_CH_EMBED, _T_CH_W, _T_CH_GAIN, _T_CH_XLAST = range(20, 24)
CHAIN_MATS = ("wq", "wk", "wv", "wo", "wg", "wu", "wd")


def chain_shapes(cfg: Config) -> dict:
    """(rows, cols) of each layer matrix (out x in) of the chain model."""
    D, I = cfg.n_q_heads * cfg.head_dim, cfg.intermediate
    kvd = cfg.n_kv_heads * cfg.head_dim
    return {"wq": (D, D), "wk": (kvd, D), "wv": (kvd, D), "wo": (D, D), "wg": (I, D), "wu": (I, D), "wd": (D, I)}


def chain_scale(cfg: Config, name: str) -> np.float32:
    """1/sqrt(fan_in) as float32: a matrix entry is bf16(N(0,1) * scale), rounded to nearest even."""
    return np.float32(1.0 / np.sqrt(chain_shapes(cfg)[name][1]))


def chain_matrix(cfg: Config, name: str, l: int) -> np.ndarray:
    """Layer l's matrix `name` (out x in), bf16 bit patterns: N(0, 1/fan_in)."""
    i = CHAIN_MATS.index(name)
    raw = _bf16_normal(_philox(cfg, _T_CH_W, i, l), chain_shapes(cfg)[name])
    return _f32_to_bf16_bits(bf16_bits_to_f32(raw) * chain_scale(cfg, name))


def chain_embed(cfg: Config) -> np.ndarray:
    """Input vector of a fed-back code, [levels-1][V][D] bf16 bit patterns, N(0, 1)."""
    D = cfg.n_q_heads * cfg.head_dim
    return _bf16_normal(_philox(cfg, _T_CH_EMBED), (max(cfg.n_levels - 1, 0), cfg.codebook, D))


def chain_gains(cfg: Config):
    """RMSNorm gains (g_attn [L][D], g_mlp [L][D], g_final [D]) float32, 1 + 0.1 N(0, 1)."""
    D, L = cfg.n_q_heads * cfg.head_dim, cfg.n_layers
    rng = np.random.default_rng(np.random.SeedSequence([cfg.seed, cfg.cfg_id, _T_CH_GAIN]))
    g = (1.0 + 0.1 * rng.standard_normal((2 * L + 1, D))).astype(np.float32)
    return g[:L], g[L:2 * L], g[2 * L]


def chain_weights(cfg: Config, layers=None) -> dict:
    """Every weight of the chain model (matrices of the listed layers, default all), host arrays:
    bf16 bit patterns for embed and the matrices [L][out][in], float32 gains."""
    layers = range(cfg.n_layers) if layers is None else layers
    w = {"embed": chain_embed(cfg)}
    for name in CHAIN_MATS:
        w[name] = np.stack([chain_matrix(cfg, name, l) for l in layers])
    w["g_attn"], w["g_mlp"], w["g_final"] = chain_gains(cfg)
    return w


def x_last(cfg: Config, r: int) -> np.ndarray:
    """Input vector of request r's last context token, [D] float32, N(0, 1)."""
    D = cfg.n_q_heads * cfg.head_dim
    return _philox(cfg, _T_CH_XLAST, r).standard_normal(D).astype(np.float32)

