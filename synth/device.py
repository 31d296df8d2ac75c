"""Device-side generation of the bf16 request inputs (libsynth_gen.so, built by synth/build.py).

The values are those of the host generators in gen.py (the same keys, the same Philox4x64-10
counter stream, the same table), written straight into device tensors, so that large
workloads need no host generation and no host-to-device copy."""
from __future__ import annotations

import ctypes
import os

import numpy as np

from .gen import (_T_CH_EMBED, _T_CH_W, _T_CTX_K, _T_CTX_V, _T_QLAST, BF16_NORMAL_TABLE, CHAIN_MATS, _key,
                  chain_gains, chain_scale, chain_shapes, request_shapes)

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsynth_gen.so")
_lib = None
_tables: dict = {}


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with synth/build.py")
        L = ctypes.CDLL(LIB_PATH)
        L.synth_bf16_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p,
                                        ctypes.c_void_p, ctypes.c_void_p]
        L.synth_bf16_normal.restype = ctypes.c_int
        _lib = L
    return _lib


def _table(device):
    import torch
    key = str(device)
    if key not in _tables:
        _tables[key] = torch.from_numpy(BF16_NORMAL_TABLE.view(np.int16)).to(device)
    return _tables[key]


def bf16_normal_into(out, key: int) -> None:
    """Fill the contiguous 2-byte device tensor `out` with the block of Philox key `key`."""
    import torch
    assert out.is_contiguous() and out.element_size() == 2 and out.is_cuda
    st = torch.cuda.current_stream(out.device).cuda_stream
    rc = lib().synth_bf16_normal(key & 0xFFFFFFFFFFFFFFFF, key >> 64, out.numel(), _table(out.device).data_ptr(),
                                 out.data_ptr(), st)
    if rc != 0:
        raise RuntimeError(f"synth_bf16_normal failed (HIP error {rc})")


def request_tensors(cfg, r: int, device="cuda"):
    """Context K, V [L][N][Hkv][d] and q_last [L][Hq][d] of request r (bf16 workloads)."""
    import torch
    assert cfg.dtype == "bf16"
    N = request_shapes(cfg)[r][0]
    L, Hkv, Hq, d = cfg.n_layers, cfg.n_kv_heads, cfg.n_q_heads, cfg.head_dim
    k = torch.empty((L, N, Hkv, d), dtype=torch.bfloat16, device=device)
    v = torch.empty((L, N, Hkv, d), dtype=torch.bfloat16, device=device)
    for l in range(L):
        bf16_normal_into(k[l], _key(cfg, _T_CTX_K, r, l))
        bf16_normal_into(v[l], _key(cfg, _T_CTX_V, r, l))
    q = torch.empty((L, Hq, d), dtype=torch.bfloat16, device=device)
    bf16_normal_into(q, _key(cfg, _T_QLAST, r))
    # the workload's power-of-two scalings (exact in bf16 for the table's range)
    if cfg.k_scale_log2:
        k.mul_(2.0 ** cfg.k_scale_log2)
    if cfg.q_scale_log2:
        q.mul_(2.0 ** cfg.q_scale_log2)
    return k, v, q


def chain_weights(cfg, device="cuda") -> dict:
    """The layer chain's weights as device tensors (gen.chain_weights' values, bit for bit): each
    matrix is drawn on the device from its Philox block, multiplied by its float32 scale and
    rounded to bf16 (nearest even), as the host generator does."""
    import torch
    L = cfg.n_layers
    D = cfg.n_q_heads * cfg.head_dim
    w = {}
    emb = torch.empty((max(cfg.n_levels - 1, 0), cfg.codebook, D), dtype=torch.bfloat16, device=device)
    if emb.numel():
        bf16_normal_into(emb, _key(cfg, _T_CH_EMBED))
    w["embed"] = emb
    for i, name in enumerate(CHAIN_MATS):
        rows, cols = chain_shapes(cfg)[name]
        out = torch.empty((L, rows, cols), dtype=torch.bfloat16, device=device)
        tmp = torch.empty((rows, cols), dtype=torch.bfloat16, device=device)
        scale = float(chain_scale(cfg, name))
        for l in range(L):
            bf16_normal_into(tmp, _key(cfg, _T_CH_W, i, l))
            out[l] = (tmp.float() * scale).to(torch.bfloat16)
        w[name] = out
    ga, gm, gf = chain_gains(cfg)
    w["g_attn"], w["g_mlp"], w["g_final"] = (torch.from_numpy(a).to(device) for a in (ga, gm, gf))
    return w

