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
from tests.engine_inputs import load_request, make_engine, native_layout, request_tensors  # noqa: F401
from tests.oracle_inputs import model_for, prefixes_for, request_for

TAU = 1e-3
SCORE_TOL = 1e-3


def attn_tol(cfg) -> float:
    return 1e-5 if cfg.dtype == "f32" else 2e-2


def gpu_beams(eng, rid):
    st = eng.state(rid)
    return [tuple(int(c) for c in row) for row in st["codes"]], st["scores"].astype(np.float64), st["parent"]


class TeacherForced:
    """Oracle bookkeeping for one request: scores of every prefix the oracle has expanded."""

    def __init__(self, cfg, r: int, norm="valid", model=None, req=None, score_tol=None, tau=None):
        self.cfg, self.r, self.norm = cfg, r, norm
        self.score_tol = SCORE_TOL if score_tol is None else score_tol
        self.tau = TAU if tau is None else tau
        self.model = model if model is not None else model_for(cfg)
        self.req = req if req is not None else request_for(cfg, r)
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
            if sc[i] > o_w + self.tau:
                assert p in chosen, f"missing beam {p} (score {sc[i]:.6f}, cutoff {o_w:.6f})"
            if sc[i] < o_w - self.tau:
                assert p not in chosen, f"extra beam {p} (score {sc[i]:.6f}, cutoff {o_w:.6f})"
        osc = np.array([self.score_of[p] for p in pref])
        dmax = float(np.max(np.abs(osc - gsc))) if len(pref) else 0.0
        assert dmax <= self.score_tol, f"score error {dmax}"
        # slot order sorted up to the band; parents consistent with prefixes
        assert np.all(osc[:-1] >= osc[1:] - self.tau), "slot order not sorted by score"
        for i, p in enumerate(pref):
            assert prev_prefixes[par[i]] == p[:-1], "parent slot does not hold the prefix"
        in_band = int(np.sum(np.abs(sc - o_w) <= self.tau))
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


def progress(msg: str):
    """Append a progress line to $GR_REPORT_DIR/progress.log when that is set (long GPU tests)."""
    import os
    import time
    d = os.environ.get("GR_REPORT_DIR")
    if d:
        os.makedirs(d, exist_ok=True)
        with open(os.path.join(d, "progress.log"), "a") as f:
            f.write(f"{time.strftime('%H:%M:%S')} {msg}\n")


def rel_err_rows(got: np.ndarray, ref: np.ndarray) -> float:
    """max over rows of max|got-ref| / max|ref| (rows = last axis)."""
    num = np.max(np.abs(got - ref), axis=-1)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return float(np.max(num / den))


def check_beam_path(eng, rid, sets):
    """BeamPath closure of a request's current beam set B_s.  sets[t] holds the code tuples of
    B_{t+1} in slot order (t < s, the last entry is B_s).  For every beam j of B_s and level t,
    anc[j][t] must be a slot of B_{t+1} whose tuple is beam j's prefix of length t+1, and the
    newest entry anc[j][s-1] is j itself (a beam's token of the latest level sits in its own
    slot)."""
    anc = eng.path(rid)
    cur, s = sets[-1], len(sets)
    assert anc.shape[0] == len(cur), (anc.shape, len(cur))
    for j, p in enumerate(cur):
        assert int(anc[j, s - 1]) == j, f"beam {j}: newest ancestor slot {anc[j, s - 1]}"
        for t in range(s):
            slot = int(anc[j, t])
            assert 0 <= slot < len(sets[t]), f"beam {j} level {t}: slot {slot} outside B_{t + 1}"
            assert sets[t][slot] == p[: t + 1], f"beam {j} level {t}: slot {slot} holds {sets[t][slot]}, not {p[:t + 1]}"


def run_checked(eng, cfg, steps, checked, attn=True, tfs=None):
    """Runs batched steps (steps: one list of request ids per gr_beam_step; ids equal the
    workload's request indices) and checks the requests in `checked` after each of their steps,
    teacher-forced: every layer's attention output of every beam (attn; needs an engine with
    debug_attn), the hidden vector, the beam set and scores, and BeamPath closure.  Returns
    (TeacherForced per checked id, attention errors, final beam sets)."""
    tfs = tfs if tfs is not None else {r: TeacherForced(cfg, r) for r in checked}
    prev = {r: [()] for r in checked}
    sets = {r: [] for r in checked}
    tol = attn_tol(cfg)
    errs = []
    for step in steps:
        eng.step(step)
        for r in step:
            if r not in tfs:
                continue
            tf = tfs[r]
            after = gpu_beams(eng, r)
            if attn:
                for l in range(cfg.n_layers):
                    got = eng.attn_out(r, l)
                    assert got.shape[0] == len(prev[r])
                    ref = np.stack([oracle.beam_layer_output(tf.req, tf.model, p, l) for p in prev[r]])
                    errs.append(rel_err_rows(got, ref))
                    assert errs[-1] <= tol, f"request {r} level {len(sets[r])} layer {l}: attention rel err {errs[-1]}"
            h, _ = eng.hidden(r)
            href = np.stack([oracle.beam_hidden(tf.req, tf.model, p) for p in prev[r]])
            assert rel_err_rows(h, href) <= tol * max(1, cfg.n_layers)
            tf.check_step(prev[r], after)
            sets[r].append(after[0])
            check_beam_path(eng, r, sets[r])
            prev[r] = after[0]
    return tfs, errs, prev


def score_bound(cfg, r: int) -> float:
    """(smallest, largest) over layers and kv heads of the Cauchy-Schwarz score bound at the
    first level: the largest |q| of the head's queries times the largest context-key norm, times
    log2(e)/sqrt(d) (the quantity the context kernels compare with their fixed-reference limit)."""
    qs = oracle.beam.as_f64(synth.q_last(cfg, r))
    g = cfg.group
    lo, hi = np.inf, 0.0
    for l in range(cfg.n_layers):
        k, _ = synth.ctx_kv_block(cfg, r, l)
        k = oracle.beam.as_f64(k)
        for h in range(cfg.n_kv_heads):
            kn = np.sqrt(np.max(np.sum(k[:, h, :] ** 2, axis=-1)))
            qn = np.max(np.linalg.norm(qs[l, h * g:(h + 1) * g, :], axis=-1))
            b = qn * kn * np.log2(np.e) / np.sqrt(cfg.head_dim)
            lo, hi = min(lo, b), max(hi, b)
    return float(lo), float(hi)
