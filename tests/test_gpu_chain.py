"""The layer chain (q/k/v/o projections, RMSNorm and SwiGLU MLP between the attention layers)
on the GPU against the float64 chain oracle.

Each kernel on its own inputs (the rows a debug engine keeps for every layer): a norm or a
projection whose output is rounded to bf16 must give the oracle's rounding of the same inputs'
exact result in all but a few elements, and those within one bf16 unit (float32 and float64
sums fall on opposite sides of a rounding boundary); a projection added into the float32
residual must agree to float32 accumulation error; layer outputs hand over exactly; the hidden
vector is the final norm of the last residual.

End to end, teacher-forced at every level: every layer's attention output of every beam (2e-2
normwise per row), the hidden vector, the beam set and the cumulative log-probs, and BeamPath
closure.  A boundary flip moves every output of the next projection by about one bf16 unit over
sqrt(K), and flips add up over the layers, so the end-to-end bound on log-probs is derived from
that arithmetic (CHAIN_SCORE_TOL) rather than the 1e-3 of the attention-only model."""
import numpy as np
import pytest

import oracle
import synth
from oracle.inputs import chain_model_for, chain_request_for
from tests.gpu_harness import TeacherForced, check_beam_path, gpu_beams, load_request, make_engine, rel_err_rows, \
    save_report

pytestmark = pytest.mark.gpu

ATTN_TOL, HIDDEN_TOL = 2e-2, 1e-2
# End to end over two layers: a boundary flip in a projection's bf16 input moves each of the
# projection's K-term outputs by about u/sqrt(K) (u = 2^-8, K >= 512: ~2e-4 relative); about one
# element per row and rounding point flips (0.05-0.2 % measured above), six points per layer, and
# the shifts add like a random walk, giving ~1e-3 relative on the hidden vector (2.2-2.3e-3
# measured) and log-prob errors of that order per level, summed over three levels and maximised
# over up to 10^5 candidates (2.4-4.5e-3 measured): 1e-2 bounds it with a factor of two.
CHAIN_SCORE_TOL = 1e-2


def _ulp(x):
    """bf16 spacing at |x| (2^(e-7) for |x| in [2^e, 2^(e+1)))."""
    a = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


def _rounded_close(got, ref_exact, window, what):
    """got (bf16 values) against the bf16 rounding of ref_exact: each element is either that
    rounding, or the rounding of a value within `window` (a bound on the float32 computation's
    error, per element) of ref_exact, i.e. |got - ref_exact| <= window + half a bf16 unit (a sum
    near a rounding boundary, or one whose float32 error exceeds the spacing after cancellation).
    Returns the fraction of elements that are not the exact rounding."""
    ref = oracle.bf16_round(ref_exact)
    ok = got == ref
    bad = ~ok & (np.abs(got - ref_exact) > window + 0.5001 * _ulp(got) + 1e-38)
    assert not np.any(bad), f"{what}: {int(np.sum(bad))} of {bad.size} elements off, e.g. got {got[bad][:3]} " \
                            f"want {ref[bad][:3]} (exact {ref_exact[bad][:3]})"
    return float(np.mean(~ok))


def _sum_err(a, w):
    """A bound on the float32 error of a @ w.T: 8 sqrt(K) 2^-24 times the sum of |terms|."""
    return 8 * np.sqrt(a.shape[-1]) * 2.0 ** -24 * (np.abs(a) @ np.abs(w).T)


def _check_kernels(eng, G, model, r, n, level, x_start):
    """The chain's kernels for request r's last step (n beams), each on its own inputs."""
    flips = []
    for l in range(model.n_layers):
        row = lambda w: eng.chain_rows(r, l, w).astype(np.float64)[:n]
        x_in, xa, q, o = row(G.GR_CHAIN_X_IN), row(G.GR_CHAIN_XN_ATTN), row(G.GR_CHAIN_Q), row(G.GR_CHAIN_O)
        x_mid, xm, act, x_out = row(G.GR_CHAIN_X_MID), row(G.GR_CHAIN_XN_MLP), row(G.GR_CHAIN_ACT), row(G.GR_CHAIN_X_OUT)
        if l == 0:
            np.testing.assert_array_equal(x_in, x_start)                       # the new tokens' input
        else:
            np.testing.assert_array_equal(x_in, prev_out)                      # layer hand-off
        flips.append(_rounded_close(xa, oracle.rms_norm(x_in, model.g_attn[l], model.eps),
                                    4e-6 * np.abs(xa) + 1e-30, f"layer {l} norm"))
        flips.append(_rounded_close(q, xa @ model.wq[l].T, _sum_err(xa, model.wq[l]), f"layer {l} q projection"))
        for name, got, ref, bound in (("output projection", x_mid - x_in, o @ model.wo[l].T, _sum_err(o, model.wo[l])),
                                      ("down projection", x_out - x_mid, act @ model.wd[l].T,
                                       _sum_err(act, model.wd[l]))):
            # the residual add rounds once more in float32
            assert np.all(np.abs(got - ref) <= bound + 2.0 ** -23 * np.abs(x_out) + 1e-30), f"layer {l} {name}"
        flips.append(_rounded_close(xm, oracle.rms_norm(x_mid, model.g_mlp[l], model.eps),
                                    4e-6 * np.abs(xm) + 1e-30, f"layer {l} mlp norm"))
        gt, up = xm @ model.wg[l].T, xm @ model.wu[l].T
        sg = 1.0 / (1.0 + np.exp(-gt))
        win = np.abs(sg * (1 + gt * (1 - sg)) * up) * _sum_err(xm, model.wg[l]) + np.abs(gt * sg) * _sum_err(xm, model.wu[l])
        flips.append(_rounded_close(act, oracle.silu(gt) * up, win + 4e-6 * np.abs(act) + 1e-30, f"layer {l} swiglu"))
        prev_out = x_out
    h, _ = eng.hidden(r)
    href = oracle.rms_norm(prev_out, model.g_final, model.eps)
    assert rel_err_rows(h[:n].astype(np.float64), href) <= 1e-5
    return max(flips)


def _cfg(**kw):
    base = dict(n_requests=2, n_layers=2, n_q_heads=4, n_kv_heads=2, head_dim=128, intermediate=1024, ctx_len=300,
                beam_width=32, n_items=5000, codebook=64)
    base.update(kw)
    return synth.get_config("chain_ctx5k_beam256_r8", **base)


def _run(cfg, steps, checked, attn_beams=None):
    """steps: request ids per batched step; checked requests are compared after each of their
    steps (attention outputs of the first attn_beams beams, default all)."""
    from semantic_id_beam_amd import _lib as G
    model = chain_model_for(cfg)
    eng = make_engine(cfg, max_requests=cfg.n_requests, debug_attn=True)
    for r in range(cfg.n_requests):
        load_request(eng, cfg, r)
    tfs = {r: TeacherForced(cfg, r, model=model, req=chain_request_for(cfg, r), score_tol=CHAIN_SCORE_TOL,
                            tau=CHAIN_SCORE_TOL) for r in checked}
    flips = []
    prev = {r: [()] for r in checked}
    sets = {r: [] for r in checked}
    errs, herrs = [], []
    for step in steps:
        eng.step(step)
        for r in step:
            if r not in tfs:
                continue
            tf = tfs[r]
            after = gpu_beams(eng, r)
            pick = prev[r][: attn_beams or len(prev[r])]
            x_start = np.stack([tf.req.x_last if len(p) == 0 else model.embed[len(p) - 1][p[-1]] for p in prev[r]])
            flips.append(_check_kernels(eng, G, model, r, len(prev[r]), len(sets[r]), x_start))
            ref = np.stack([oracle.chain_layer_outputs(tf.req, model, p) for p in pick])   # [n][L][Hq][d]
            for l in range(cfg.n_layers):
                got = eng.attn_out(r, l)[: len(pick)]
                errs.append(rel_err_rows(got, ref[:, l]))
                assert errs[-1] <= ATTN_TOL, f"request {r} level {len(sets[r])} layer {l}: attention rel err {errs[-1]}"
            h, _ = eng.hidden(r)
            href = np.stack([oracle.chain_hidden(tf.req, model, p) for p in pick])
            herrs.append(rel_err_rows(h[: len(pick)], href))
            assert herrs[-1] <= HIDDEN_TOL, f"request {r} level {len(sets[r])}: hidden rel err {herrs[-1]}"
            tf.check_step(prev[r], after)
            sets[r].append(after[0])
            check_beam_path(eng, r, sets[r])
            prev[r] = after[0]
    final = {r: eng.beams(r) for r in checked}
    for r in checked:
        assert [tuple(c) for c in final[r][0].tolist()] == prev[r]
    eng.close()
    save_report(cfg, [x for r in checked for x in tfs[r].report], attn_err=max(errs), hidden_err=max(herrs),
                max_flip_fraction=max(flips))
    return final


def test_chain_small_lockstep_matches_oracle():
    cfg = _cfg()
    a = _run(cfg, [[0, 1]] * cfg.n_levels, [0, 1])
    # deterministic: the same decode again, bit for bit
    b = _run(cfg, [[0, 1]] * cfg.n_levels, [1])
    assert np.array_equal(a[1][0], b[1][0]) and np.array_equal(a[1][1].view(np.uint32), b[1][1].view(np.uint32))


def test_chain_every_attention_variant_mixed_levels():
    """Beam widths 8, 30, 50 and 150 (one- and two-wave stream kernels, the four-wave narrow
    kernel, the wide kernel), ragged contexts, admitted in two waves so that the middle steps
    pack rows of levels 0, 1 and 2 together."""
    shapes = ((300, 8), (513, 30), (257, 50), (190, 150), (64, 30), (700, 8))
    cfg = _cfg(n_requests=6, shapes=shapes, waves=2)
    steps = [[0, 1, 2], [0, 1, 2, 3, 4, 5], [0, 1, 2, 3, 4, 5], [3, 4, 5]]
    _run(cfg, steps, [0, 2, 3, 5], attn_beams=40)


def test_chain_head_dim_64():
    cfg = _cfg(n_q_heads=4, n_kv_heads=2, head_dim=64, intermediate=512, beam_width=16)
    _run(cfg, [[0, 1]] * cfg.n_levels, [1])


@pytest.mark.timeout(600)
def test_chain_qwen3_shape_two_layers():
    """Qwen3-1.7B's layer shape (hidden 2048, 16/8 heads of 128, MLP 6144) over two layers (weights
    drawn on the device), 32 beams per request; the first 8 beams' attention outputs and hidden
    vectors are checked, every candidate score of every beam."""
    cfg = _cfg(n_q_heads=16, n_kv_heads=8, head_dim=128, intermediate=6144, ctx_len=500, beam_width=32, n_items=50000,
               codebook=256)
    _run(cfg, [[0, 1]] * cfg.n_levels, [1], attn_beams=8)
