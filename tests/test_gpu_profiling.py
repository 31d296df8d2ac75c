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


def test_wave_timeline_build_records_every_wave_in_order():
    # bench.py --wave-times: a child process with the wave-timeline build records one headline
    # launch (level 1, layer 13); every wave's stamps must be present and ordered
    import json
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    if not os.path.exists(os.path.join(root, "semantic_id_beam_amd", "libgr_beam_timed.so")):
        pytest.fail("libgr_beam_timed.so is missing: build the package first")
    print("wave timeline: bench.py --wave-times (headline, level 1, layer 13)", flush=True)
    res = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--wave-times"], cwd=root,
                         stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=110)
    assert res.returncode == 0, res.stderr[-2000:]
    wt = json.loads(res.stdout.strip().splitlines()[-1])["wave_times"]
    assert wt["workgroups"] == 256 and wt["waves"] == 2048  # 8 requests x 8 kv heads x 2 splits x 2 row blocks
    assert 0 < wt["prologue_us"]["median"] <= wt["prologue_us"]["max"]
    assert 0 < wt["loop_us"]["min"] <= wt["loop_us"]["median"] <= wt["loop_us"]["max"]
    assert 0 < wt["epilogue_us"]["median"] <= wt["epilogue_us"]["max"]
    assert wt["span_us"] >= wt["loop_us"]["max"]
    assert len(wt["xcd_median_end_us"]) == 8
    assert 0 < wt["loop_copy_wait_frac"] < 1 and 0 < wt["loop_barrier_frac"] < 1
    assert wt["loop_copy_wait_frac"] + wt["loop_barrier_frac"] < 1
    assert wt["barriers_per_wave"] >= 30  # about one per 64-token tile of a 2,500-token range
