"""Launch profiling on the GPU: sampled per-layer events (gr_engine_set_profiling_stride) time
only the chosen layers' launches and leave the decode's results unchanged."""
import numpy as np
import pytest

import synth
from tests.gpu_harness import load_request, make_engine

pytestmark = pytest.mark.gpu


def test_profiling_stride_times_every_kth_layer():
    import semantic_id_beam_amd._lib as G
    cfg = synth.get_config("ctx1k_beam256", n_requests=2, n_layers=5, ctx_len=300, beam_width=64, n_items=50000)
    plain = make_engine(cfg, max_requests=2, per_layer=True)
    prof = make_engine(cfg, max_requests=2, per_layer=True)
    rids = [load_request(plain, cfg, r) for r in range(2)]
    assert [load_request(prof, cfg, r) for r in range(2)] == rids
    G.gr_engine_profile_reset(prof.eng)
    G.gr_engine_set_profiling_kinds(prof.eng, 1 << G.GR_PROF_CTX_ATTN)
    G.gr_engine_set_profiling_stride(prof.eng, 2)
    for s in range(cfg.n_levels):
        plain.step(rids)
        prof.step(rids)
    G.gr_engine_set_profiling(prof.eng, False)
    for s in range(cfg.n_levels):
        # layers 0, 2 and 4 of the five carry events, one launch each (one variant group)
        assert G.gr_engine_profile_dispatches(prof.eng, G.GR_PROF_CTX_ATTN, s) == 3, s
        ms, launches = G.gr_engine_profile_read(prof.eng, G.GR_PROF_CTX_ATTN, s)
        assert launches == 3 and ms > 0.0, (s, ms, launches)
        _, merges = G.gr_engine_profile_read(prof.eng, G.GR_PROF_BEAM_MERGE, s)
        assert merges == 0
    for r in rids:
        ca, sa = plain.beams(r)
        cb, sb = prof.beams(r)
        assert np.array_equal(ca, cb) and np.array_equal(sa.view(np.uint32), sb.view(np.uint32))
    plain.close()
    prof.close()
