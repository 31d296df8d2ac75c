"""Continuous batching through the host scheduler (gr_sched_*), on the GPU.

Requests arrive two per scheduling round into a scheduler that decodes at most six at once,
so every batched step mixes requests at different levels, some join and some leave.  The
scheduler's results are checked against the engine driven directly with the same step
compositions (FIFO admission, one step per round: replayed here), bit for bit, and sampled
final scores against the oracle's item scores (the sum of per-level constrained log-probs
along each returned code tuple)."""
from collections import deque

import numpy as np
import pytest

import oracle
import semantic_id_beam_amd as sib
import synth
from tests.engine_inputs import make_engine, request_tensors
from tests.gpu_harness import SCORE_TOL, save_report
from tests.oracle_inputs import model_for, prefixes_for, request_for

pytestmark = pytest.mark.gpu

MAX_ACTIVE = 6


def _cfg():
    # ragged contexts and beam widths; 5 levels, Zipf item set
    shapes = ((300, 30), (257, 30), (130, 12), (700, 30), (64, 5), (333, 30), (1, 30), (520, 20),
              (300, 30), (191, 30), (65, 30), (444, 8), (300, 30), (129, 30), (600, 30), (77, 30))
    return synth.get_config("ctx2k_beam30_r64", n_requests=len(shapes), n_layers=3, shapes=shapes,
                            n_items=40000)


def test_scheduler_matches_replayed_steps_and_oracle():
    cfg = _cfg()
    R, lv = cfg.n_requests, cfg.n_levels
    shapes = synth.request_shapes(cfg)
    tens = {r: request_tensors(cfg, r) for r in range(R)}

    eng = make_engine(cfg, max_requests=MAX_ACTIVE + 2)
    sched = sib.Scheduler(eng, MAX_ACTIVE)
    rounds, results, nxt = [], {}, 0
    with pytest.raises(sib.GrError):
        sched.result(0)                                    # nothing finished yet
    while len(results) < R:
        subs = []
        for _ in range(2):
            if nxt < R:
                k, v, q = tens[nxt]
                sched.submit(nxt, k, v, q, shapes[nxt][1])
                subs.append(nxt)
                nxt += 1
        if subs:
            with pytest.raises(sib.GrError):
                sched.submit(subs[0], *tens[subs[0]], shapes[subs[0]][1])   # id already queued
        rounds.append(subs)
        sched.advance()
        for rid in sched.completed():
            results[int(rid)] = sched.result(int(rid))
        assert len(rounds) < 200
    counts = sched.counts()
    assert counts == {"queued": 0, "active": 0, "done": 0, "steps": counts["steps"]}
    assert sched.flush() == 0
    sched.close()
    eng.close()

    # replay: FIFO admission up to MAX_ACTIVE, one step per round, the engine called directly
    eng2 = make_engine(cfg, max_requests=MAX_ACTIVE + 2)
    queue, active, level, ref, sizes = deque(), [], {}, {}, []
    for subs in rounds:
        queue.extend(subs)
        while queue and len(active) < MAX_ACTIVE:
            r = queue.popleft()
            eng2.load(r, *tens[r], shapes[r][1])
            active.append(r)
            level[r] = 0
        if not active:
            continue
        sizes.append(len(active))
        eng2.step(active)
        for r in active:
            level[r] += 1
        for r in [r for r in active if level[r] == lv]:
            ref[r] = eng2.beams(r)
            eng2.release(r)
        active = [r for r in active if level[r] < lv]
    eng2.close()
    assert len(sizes) == counts["steps"]
    assert max(sizes) == MAX_ACTIVE and len(set(sizes)) > 1
    for r in range(R):
        (c0, s0), (c1, s1) = results[r], ref[r]
        assert np.array_equal(c0, c1) and np.array_equal(s0, s1), r

    # oracle: each returned beam is an item and its score is the item's log-probability
    model, ps = model_for(cfg), prefixes_for(cfg)
    worst = 0.0
    for r in (2, 7, 13):
        codes, scores = results[r]
        assert codes.shape[0] == min(shapes[r][1], len(ps.levels[lv]))
        assert np.all(scores[:-1] >= scores[1:])
        for it in codes:
            assert ps.contains(tuple(int(x) for x in it))
        want = oracle.score_items(request_for(cfg, r), model, ps, codes)
        worst = max(worst, float(np.max(np.abs(want - scores))))
    assert worst <= SCORE_TOL, worst
    save_report(cfg, [], sched_steps=counts["steps"], score_err=worst)
