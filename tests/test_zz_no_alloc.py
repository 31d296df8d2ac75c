"""The allocation-free prefill (gr_ctx_prefill_noalloc) against gr_ctx_prefill.

Both run the same kernels on the same token ids (device memory for the former, host memory for
the latter) and the same soft token; the soft token's partial sums go to the library's fixed
device array in one case and to the engine's staging in the other.  The native K, V^T and the
last query must agree bit for bit, and so must a decode of each request.  Two calls in a row on
the same GPU, the second with a shorter context and the soft token in last place (the fixed
array keeps the first call's contents, which the second must fully overwrite), then a third
without a soft token.  A model whose soft-token partial sums do not fit the array is refused."""
import numpy as np
import pytest

import synth
from semantic_id_beam_amd import _lib as G
from semantic_id_beam_amd.workloads import make_engine

pytestmark = pytest.mark.gpu

VOCAB, DU, DE = 500, 24, 200


def _native(cfg, N, fill):
    import torch
    Np = (N + 63) // 64 * 64
    L, H, d = cfg.n_layers, cfg.n_kv_heads, cfg.head_dim
    return (torch.full((L, H, Np, d), fill, dtype=torch.bfloat16, device="cuda"),
            torch.full((L, H, d, Np), fill, dtype=torch.bfloat16, device="cuda"),
            torch.full((L, cfg.n_q_heads, d), fill, dtype=torch.bfloat16, device="cuda"))


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy()


def test_prefill_noalloc_equals_prefill():
    import torch
    cfg = synth.get_config("ctx1k_beam256", n_layers=3, ctx_len=300, beam_width=32, n_items=5000)
    tabs = synth.prefill_tables(cfg, VOCAB)
    soft = synth.soft_token_weights(cfg, DU, DE)
    eng = make_engine(cfg, max_requests=2, max_ctx_tokens=0)
    eng.set_prefill(*tabs, *soft)
    W = 32
    for call, (N, soft_pos) in enumerate([(300, 17), (130, 129), (97, -1)]):
        toks = synth.prefill_tokens(cfg, call, VOCAB, N)
        user = torch.from_numpy(synth.user_vector(cfg, call, DU)).cuda()
        ka, va, qa = _native(cfg, N, 3.0)
        kb, vb, qb = _native(cfg, N, -5.0)
        eng.prefill(10, toks, W, soft_pos=soft_pos, user_vec=user if soft_pos >= 0 else None,
                    k_native=ka, vt_native=va, q_last_out=qa)
        eng.prefill_noalloc(11, torch.from_numpy(toks).cuda(), W, soft_pos=soft_pos,
                            user_vec=user if soft_pos >= 0 else None, k_native=kb, vt_native=vb, q_last_out=qb)
        torch.cuda.synchronize()
        for a, b in ((ka, kb), (va, vb), (qa, qb)):
            assert np.array_equal(_bits(a), _bits(b)), f"call {call}: native layout differs"
        for _ in range(cfg.n_levels):
            eng.step([10, 11])
        (ca, sa), (cb, sb) = eng.beams(10), eng.beams(11)
        assert np.array_equal(ca, cb) and np.array_equal(sa.view(np.uint32), sb.view(np.uint32)), call
        assert ca.shape[0] == W
        eng.release(10)
        eng.release(11)
    eng.close()


def test_prefill_noalloc_refuses_oversized_soft_token():
    """28 layers of 32 query / 4 kv heads of 128: 8 partial sums of 64 + 28 * 5120 floats are
    4.6 MB, more than the 4 MiB array; the same model without a soft token prefills."""
    import torch
    cfg = synth.get_config("ctx1k_beam256", n_layers=28, n_q_heads=32, n_kv_heads=4, ctx_len=64, beam_width=4,
                           n_items=1000)
    tabs = synth.prefill_tables(cfg, 16)
    soft = synth.soft_token_weights(cfg, 8, 64)
    eng = make_engine(cfg, max_requests=1, max_ctx_tokens=64)
    eng.set_prefill(*tabs, *soft)
    toks = torch.arange(64, dtype=torch.int32, device="cuda") % 16
    user = torch.ones(8, dtype=torch.float32, device="cuda")
    with pytest.raises(G.GrError) as ei:
        eng.prefill_noalloc(1, toks, 4, soft_pos=5, user_vec=user)
    assert ei.value.status == G.GR_E_UNSUPPORTED
    eng.prefill_noalloc(1, toks, 4)
    for _ in range(cfg.n_levels):
        eng.step([1])
    codes, _ = eng.beams(1)
    assert codes.shape[0] == 4
    eng.close()
