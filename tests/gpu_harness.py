"""GPU-side helpers for the parity tests: build engines from the seeded inputs
and compare the HIP path with the oracle step by step (teacher-forced).

Matching rules (the method's tolerance statement, restated):
  * surviving sets and BeamPath indices are exact wherever neighbouring oracle
    scores differ by more than TAU = 1e-3;
  * cumulative log-probs within 1e-3 absolute;
  * attention outputs within 1e-5 (float32 model) or 2e-2 (bf16 K/V, fp32
    accumulate) relative, normwise per (beam, query head) row:
    max|o - o_ref| / max|o_ref|.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth
from tests.oracle_inputs import model_for, prefixes_for, request_for

TAU = 1e-3
SCORE_TOL = 1e-3


def attn_tol(cfg) -> float:
    return 1e-5 if cfg.dtype == "f32" else 2e-2


def make_engine(cfg, *, max_requests=None, max_splits=0, debug_attn=False, norm="valid", max_ctx_tokens=None,
                max_beam_width=None):
    import semantic_id_beam_amd as sib
    tq, tk, tv = synth.token_tables(cfg)
    shapes = synth.request_shapes(cfg)
    R = cfg.n_requests if max_requests is None else max_requests
    if max_ctx_tokens is None:
        max_ctx_tokens = sum(sib._lib.lib().gr_ctx_padded_len(n) for n, _ in shapes[:R])
    W = max(w for _, w in shapes) if max_beam_width is None else max_beam_width
    return sib.BeamEngine(tok_q=tq, tok_k=tk, tok_v=tv, w_sid=synth.w_sid(cfg), items=synth.items(cfg),
                          n_layers=cfg.n_layers, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                          head_dim=cfg.head_dim, dtype=cfg.dtype, norm=norm, max_requests=R,
                          max_beam_width=W, max_ctx_tokens=max_ctx_tokens, max_splits=max_splits,
                          debug_attn=debug_attn)


def request_tensors(cfg, r: int, device="cuda"):
    """Context K, V [L][N][Hkv][d] and q_last [L][Hq][d] of request r as device tensors."""
    from semantic_id_beam_amd import to_device
    ks, vs = [], []
    for l in range(cfg.n_layers):
        k, v = synth.ctx_kv_block(cfg, r, l)
        ks.append(k)
        vs.append(v)
    return to_device(np.stack(ks), device), to_device(np.stack(vs), device), to_device(synth.q_last(cfg, r), device)


def native_layout(k, v):
    """[L][N][Hkv][d] -> (K [L][Hkv][Np][d], V^T [L][Hkv][d][Np]) zero-padded (test-side data prep)."""
    import torch
    L, N, Hkv, d = k.shape
    Np = (N + 63) // 64 * 64
    kn = torch.zeros((L, Hkv, Np, d), dtype=k.dtype, device=k.device)
    vn = torch.zeros((L, Hkv, d, Np), dtype=v.dtype, device=v.device)
    kn[:, :, :N, :] = k.permute(0, 2, 1, 3)
    vn[:, :, :, :N] = v.permute(0, 2, 3, 1)
    return kn.contiguous(), vn.contiguous(), N


def load_request(eng, cfg, r: int, rid: int | None = None, adopt=False):
    k, v, q = request_tensors(cfg, r)
    N, W = synth.request_shapes(cfg)[r]
    rid = r if rid is None else rid
    if adopt:
        kn, vn, _ = native_layout(k, v)
        eng.load(rid, kn, vn, q, W, adopt=True, ctx_len=N)
    else:
        eng.load(rid, k, v, q, W)
    return rid


def gpu_beams(eng, rid):
    st = eng.state(rid)
    return [tuple(int(c) for c in row) for row in st["codes"]], st["scores"].astype(np.float64), st["parent"]


class TeacherForced:
    """Oracle bookkeeping for one request: scores of every prefix the oracle has expanded."""

    def __init__(self, cfg, r: int, norm="valid"):
        self.cfg, self.r, self.norm = cfg, r, norm
        self.model = model_for(cfg)
        self.req = request_for(cfg, r)
        self.ps = prefixes_for(cfg)
        self.score_of = {(): 0.0}
        self.W = synth.request_shapes(cfg)[r][1]
        self.report = []

    def check_step(self, prev_prefixes, gpu_after):
        """prev_prefixes: GPU beam set B_s (slot order); gpu_after: (prefixes, scores, parents) of B_{s+1}."""
        V = self.cfg.codebook
        beams = [(p, self.score_of[p]) for p in prev_prefixes]
        sc, js, cs = oracle.step_candidates(self.req, self.model, self.ps, beams, self.norm)
        for s_, j_, c_ in zip(sc, js, cs):
            self.score_of[prev_prefixes[j_] + (int(c_),)] = float(s_)
        n_exp = min(self.W, sc.shape[0])
        pref, gsc, par = gpu_after
        assert len(pref) == n_exp, f"beam count {len(pref)} != {n_exp}"
        order = oracle.select_topk(sc, js, cs, self.W, V)
        o_w = sc[order[-1]]
        chosen = set(pref)
        assert len(chosen) == len(pref), "duplicate beams"
        # must-have / must-not sets outside the tie band
        for i in range(sc.shape[0]):
            p = prev_prefixes[js[i]] + (int(cs[i]),)
            if sc[i] > o_w + TAU:
                assert p in chosen, f"missing beam {p} (score {sc[i]:.6f}, cutoff {o_w:.6f})"
            if sc[i] < o_w - TAU:
                assert p not in chosen, f"extra beam {p} (score {sc[i]:.6f}, cutoff {o_w:.6f})"
        osc = np.array([self.score_of[p] for p in pref])
        dmax = float(np.max(np.abs(osc - gsc))) if len(pref) else 0.0
        assert dmax <= SCORE_TOL, f"score error {dmax}"
        # slot order sorted up to the band; parents consistent with prefixes
        assert np.all(osc[:-1] >= osc[1:] - TAU), "slot order not sorted by score"
        for i, p in enumerate(pref):
            assert prev_prefixes[par[i]] == p[:-1], "parent slot does not hold the prefix"
        in_band = int(np.sum(np.abs(sc - o_w) <= TAU))
        exact = [prev_prefixes[js[i]] + (int(cs[i]),) for i in order] == list(pref)
        self.report.append({"n": n_exp, "max_dscore": dmax, "in_band": in_band, "exact_order": exact})
        return self.report[-1]


def save_report(cfg, steps, **extra):
    """Append a parity report line to $GR_REPORT_DIR/parity_reports.jsonl when that is set."""
    import json
    import os
    d = os.environ.get("GR_REPORT_DIR")
    if not d:
        return
    os.makedirs(d, exist_ok=True)
    test = os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0]
    with open(os.path.join(d, "parity_reports.jsonl"), "a") as f:
        f.write(json.dumps({"test": test, "config": cfg.name, "steps": steps, **extra}) + "\n")


def rel_err_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max|got-ref| / max|ref| (rows = last axis)."""
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den))
