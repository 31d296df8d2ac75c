"""Graph replay of decode steps (GR_ENGINE_GRAPH) against the same engine launching directly.

Every step of a graph engine is compared bit for bit with an engine that launches the same
sequence directly (beam codes, scores, parents and BeamPath), over decodes repeated after
resets, with the program's own eager work (result gathers, resets, a device reduction) and
synchronisations between the replays; the graph counters show that later decodes replay the
graphs captured by the first."""
import numpy as np
import pytest

import synth
from tests.gpu_harness import load_request, make_engine

pytestmark = pytest.mark.gpu


def _same_state(a, b, rids):
    for r in rids:
        sa, sb = a.state(r), b.state(r)
        for k in ("codes", "scores", "parent"):
            x, y = np.ascontiguousarray(sa[k]), np.ascontiguousarray(sb[k])
            assert x.shape == y.shape and np.array_equal(x.view(np.uint8), y.view(np.uint8)), (r, k)
        s = sa["level"]  # anc[j][t] is defined for t < s
        assert np.array_equal(a.path(r)[:, :s], b.path(r)[:, :s]), r


@pytest.mark.parametrize("per_layer", [True, False])
def test_lockstep_decodes_replay_bit_identically(per_layer):
    import torch
    import semantic_id_beam_amd._lib as G
    cfg = synth.get_config("ctx1k_beam256", n_requests=4, n_layers=3, ctx_len=700, beam_width=200, n_items=50000)
    eager = make_engine(cfg, max_requests=4, per_layer=per_layer)
    graph = make_engine(cfg, max_requests=4, per_layer=per_layer, graph=True)
    rids = [load_request(eager, cfg, r) for r in range(4)]
    assert [load_request(graph, cfg, r) for r in range(4)] == rids
    reps = 3
    for rep in range(reps):
        for s in range(cfg.n_levels):
            eager.step(rids)
            graph.step(rids)
            _same_state(eager, graph, rids)
            # eager work and a synchronisation between the replays
            x = torch.arange(1 << 16, device="cuda", dtype=torch.float32)
            assert float(x.sum()) == float((1 << 16) * ((1 << 16) - 1) // 2)
            torch.cuda.synchronize()
        for r in rids:
            ce, se = eager.beams(r)
            cg, sg = graph.beams(r)
            assert np.array_equal(ce, cg) and np.array_equal(se.view(np.uint32), sg.view(np.uint32))
        eager.reset_batch(rids)
        graph.reset_batch(rids)
    # level 0 has its own shape; levels 1 and 2 both hold beam_width beams per request, so their
    # steps share one graph
    captures, replays = G.gr_engine_graph_stats(graph.eng)
    assert captures == 2 and captures + replays == cfg.n_levels * reps, (captures, replays)
    eager.close()
    graph.close()


def test_continuous_batching_steps_replay_bit_identically():
    """Requests admitted in two waves, so steps mix levels (several variant groups on the engine's
    streams inside one graph); the whole schedule runs twice."""
    import semantic_id_beam_amd._lib as G
    wave = ((333, 30),) * 3 + ((333, 150), (129, 5))
    shapes = wave + tuple((n + 40, w) for n, w in wave)
    cfg = synth.get_config("ragged_r128", n_requests=len(shapes), n_layers=2, shapes=shapes, n_items=60000, waves=2)
    R = cfg.n_requests
    eager = make_engine(cfg, max_requests=R)
    graph = make_engine(cfg, max_requests=R, graph=True)
    for e in (eager, graph):
        for r in range(R):
            load_request(e, cfg, r)
    waves = [list(range(5)), list(range(5, 10))]
    for rep in range(2):
        level = {}
        for k in range(len(waves) + cfg.n_levels - 1):
            if k < len(waves):
                for r in waves[k]:
                    level[r] = 0
            step = [r for r in level if level[r] < cfg.n_levels]
            eager.step(step)
            graph.step(step)
            _same_state(eager, graph, step)
            for r in step:
                level[r] += 1
        eager.reset_batch(list(range(R)))
        graph.reset_batch(list(range(R)))
    # every step of the second pass replays a graph of the first
    n_steps = len(waves) + cfg.n_levels - 1
    captures, replays = G.gr_engine_graph_stats(graph.eng)
    assert captures <= n_steps and captures + replays == 2 * n_steps and replays >= n_steps, (captures, replays)
    eager.close()
    graph.close()
