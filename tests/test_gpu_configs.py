"""Parity at the full workload sizes, in the launch configuration bench.py times.

Every request of a workload is loaded and stepped together (the ragged workload in its
four admission waves), exactly as the benchmark runs them.  The oracle is too slow to
recompute every beam at these sizes, so it checks sampled outputs one by one:

  * hidden vectors of sampled beams after each step (attention tolerance, normwise);
  * every candidate of sampled parent beams: children the GPU kept must carry
    parent score + oracle log-prob within 1e-3, and the GPU's cut must respect the
    oracle scores outside a +-1e-3 band;
  * cumulative log-probs of sampled final beams recomputed level by level (1e-3);

and properties that hold at any size check every request: each final beam is a valid
item, scores are sorted, and the beam count is min(W, reachable items).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.engine_inputs import make_engine, request_tensors
from tests.gpu_harness import SCORE_TOL, TAU, attn_tol, progress, rel_err_rows, save_report
from tests.oracle_inputs import model_for, prefixes_for, request_for

pytestmark = pytest.mark.gpu


class OracleSampler:
    """Oracle log-probs of single prefixes of one request, cached."""

    def __init__(self, cfg, r):
        self.cfg, self.model, self.ps = cfg, model_for(cfg), prefixes_for(cfg)
        self.req = request_for(cfg, r)
        self.cache = {}
        self.hcache = {}

    def hidden(self, prefix):
        if prefix not in self.hcache:
            self.hcache[prefix] = oracle.beam_hidden(self.req, self.model, prefix)
        return self.hcache[prefix]

    def logp(self, prefix):
        """{code: log-prob} over the valid codes after `prefix`."""
        if prefix not in self.cache:
            valid = self.ps.valid_codes(prefix)
            lg = oracle.codebook_logits(self.model, self.hidden(prefix), len(prefix))
            lp = oracle.constrained_log_softmax(lg, valid, "valid")
            self.cache[prefix] = dict(zip(valid.tolist(), lp.tolist()))
        return self.cache[prefix]

    def score(self, item):
        return sum(self.logp(tuple(item[:t]))[int(item[t])] for t in range(len(item)))


def _check_step(orc, before, after, W, n_parents, rng, tol, stats):
    """before/after: GPU beam states around one step of one request."""
    prefixes = [tuple(int(c) for c in row) for row in before["codes"]]
    kids = [tuple(int(c) for c in row) for row in after["codes"]]
    kid_score = dict(zip(kids, after["scores"].astype(np.float64)))
    cut = float(after["scores"][-1]) if len(kids) >= W else -np.inf
    pick = rng.choice(len(prefixes), size=min(n_parents, len(prefixes)), replace=False)
    for j in pick:
        p = prefixes[j]
        for c, lp in orc.logp(p).items():
            s = float(before["scores"][j]) + lp
            child = p + (c,)
            if child in kid_score:
                stats["step"] = max(stats["step"], abs(kid_score[child] - s))
                assert abs(kid_score[child] - s) <= SCORE_TOL, (child, kid_score[child], s)
            elif s > cut + TAU:
                raise AssertionError(f"candidate {child} (score {s:.6f}) above the cut {cut:.6f} was dropped")
            if child in kid_score and s < cut - TAU:
                raise AssertionError(f"candidate {child} (score {s:.6f}) below the cut {cut:.6f} was kept")
    return pick


def _check_hidden(orc, eng, rid, before, pick, tol, stats):
    h, _ = eng.hidden(rid)
    prefixes = [tuple(int(c) for c in row) for row in before["codes"]]
    ref = np.stack([orc.hidden(prefixes[j]) for j in pick])
    err = rel_err_rows(h[pick], ref)
    stats["hidden"] = max(stats["hidden"], err)
    assert err <= tol, f"hidden rel err {err}"


def _final_properties(cfg, ps, codes, scores, W):
    items = {tuple(int(x) for x in row) for row in codes}
    assert len(items) == codes.shape[0]
    for it in items:
        assert ps.contains(it)
    assert np.all(scores[:-1] >= scores[1:])
    # reachable items bound the count
    assert codes.shape[0] == min(W, len(ps.levels[cfg.n_levels]))


def _run_full(cfg, sampled, schedule=None, n_parents=2, n_final=3):
    """Decode every request of cfg as the benchmark does; check `sampled` requests against the oracle."""
    shapes = synth.request_shapes(cfg)
    R, lv = cfg.n_requests, cfg.n_levels
    eng = make_engine(cfg, max_requests=R)
    tol = attn_tol(cfg)
    rng = np.random.default_rng(7)
    orcs = {r: OracleSampler(cfg, r) for r in sampled}
    ps = prefixes_for(cfg)
    stats = {"step": 0.0, "hidden": 0.0, "final": 0.0}
    if schedule is None:
        schedule = [list(range(R))]                      # one admission wave
    waves = list(schedule)
    level = {}
    done = {}
    admitted = []
    k = 0
    while waves or any(level[r] < lv for r in admitted):
        if waves:                                        # admit the next wave before this step
            for r in waves.pop(0):
                kk, vv, qq = request_tensors(cfg, r)
                eng.load(r, kk, vv, qq, shapes[r][1])
                del kk, vv, qq
                level[r] = 0
                admitted.append(r)
                if len(admitted) % 16 == 0:
                    progress(f"{cfg.name}: loaded {len(admitted)} requests")
        step = [r for r in admitted if level[r] < lv]
        before = {r: eng.state(r) for r in step if r in orcs}
        eng.step(step)
        k += 1
        progress(f"{cfg.name}: batched step {k} over {len(step)} requests")
        for r in step:
            level[r] += 1
            if r in orcs:
                after = eng.state(r)
                pick = _check_step(orcs[r], before[r], after, shapes[r][1], n_parents, rng, tol, stats)
                _check_hidden(orcs[r], eng, r, before[r], pick, tol, stats)
                progress(f"{cfg.name}: request {r} level {level[r]} checked against the oracle")
            if level[r] == lv:
                codes, scores = eng.beams(r)
                _final_properties(cfg, ps, codes, scores, shapes[r][1])
                if r in orcs:
                    for i in rng.choice(codes.shape[0], size=min(n_final, codes.shape[0]), replace=False):
                        want = orcs[r].score(codes[i])
                        stats["final"] = max(stats["final"], abs(float(scores[i]) - want))
                        assert abs(float(scores[i]) - want) <= SCORE_TOL, (r, codes[i], scores[i], want)
                done[r] = True
                eng.release(r)
    eng.close()
    assert len(done) == R
    save_report(cfg, [], **stats)
    return k


@pytest.mark.timeout(900)
@pytest.mark.timeout(900)
def test_headline_ctx5k_beam256_r8_full():
    cfg = synth.get_config("ctx5k_beam256_r8")
    steps = _run_full(cfg, sampled=[0, 2, 5, 7], n_parents=4, n_final=4)
    assert steps == cfg.n_levels


@pytest.mark.timeout(900)
def test_ctx2k_beam30_r64_zipf_full():
    cfg = synth.get_config("ctx2k_beam30_r64")
    steps = _run_full(cfg, sampled=[3, 17, 41, 60], n_parents=3)
    assert steps == cfg.n_levels


@pytest.mark.timeout(1200)
def test_ragged_r128_four_waves_full():
    cfg = synth.get_config("ragged_r128")
    R = cfg.n_requests
    per = R // cfg.waves
    schedule = [list(range(w * per, (w + 1) * per)) for w in range(cfg.waves)]
    shapes = synth.request_shapes(cfg)
    # sample one request per wave with a beam width not sampled yet
    sampled, seen = [], set()
    for wave in schedule:
        for r in wave:
            if shapes[r][1] not in seen:
                seen.add(shapes[r][1])
                sampled.append(r)
                break
    steps = _run_full(cfg, sampled=sampled, schedule=schedule)
    assert steps == cfg.waves + cfg.n_levels - 1          # 6 batched steps: 32/64/96/96/64/32 requests
