"""The device generator of the bf16 inputs gives the host generators' values, bit for bit."""
import numpy as np
import pytest

import synth
from synth.gen import _T_CTX_K, _key, _philox, _bf16_normal

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(dtype=__import__("torch").int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n", [1, 15, 16, 17, 4096 + 5, 1 << 20])
def test_block_lengths(n):
    import torch
    from synth import device as sd
    cfg = synth.get_config("ragged_r128")
    out = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    sd.bf16_normal_into(out, _key(cfg, _T_CTX_K, 9, 4))
    want = _bf16_normal(_philox(cfg, _T_CTX_K, 9, 4), (n,))
    assert np.array_equal(_bits(out), want)


@pytest.mark.parametrize("name,r", [("ctx1k_beam256", 0), ("ragged_r128", 77), ("ctx2k_beam30_r64", 63)])
def test_request_tensors_equal_host(name, r):
    from tests.engine_inputs import request_tensors
    cfg = synth.get_config(name, n_layers=3) if name != "ctx1k_beam256" else synth.get_config(name)
    dk, dv, dq = request_tensors(cfg, r)
    hk, hv, hq = request_tensors(cfg, r, host=True)
    for a, b in ((dk, hk), (dv, hv), (dq, hq)):
        assert a.shape == b.shape and a.dtype == b.dtype
        assert np.array_equal(_bits(a), _bits(b))


def test_chain_weights_equal_host():
    """The layer chain's weights drawn on the device (scaled and rounded to bf16 there) equal the
    host generator's, bit for bit, at Qwen3-1.7B's layer shape."""
    from synth import device as sd
    cfg = synth.get_config("chain_ctx5k_beam256_r8", n_layers=2)
    dw = sd.chain_weights(cfg)
    hw = synth.chain_weights(cfg)
    for k in ("embed",) + synth.CHAIN_MATS:
        assert tuple(dw[k].shape) == hw[k].shape, k
        assert np.array_equal(_bits(dw[k]), hw[k]), k
    for k in ("g_attn", "g_mlp", "g_final"):
        assert np.array_equal(dw[k].cpu().numpy(), hw[k]), k
