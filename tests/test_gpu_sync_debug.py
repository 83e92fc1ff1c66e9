"""KDA_SYNC_DEBUG: with it set, the entry points wait for their stream
before returning; their results must be those of the asynchronous calls
(prefill one-pass and segmented, decode, backward)."""
import pytest
import torch

import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_61_amd as kda
    kda.lib()
    return kda


def _calls(kda):
    inp = W.prefill_inputs(W.PREFILL_BF16_H16_T4K, device="cuda", B=1, T=64 * 30 + 5, H=2, seed=71)
    B, T, H, _ = inp["q"].shape
    need = kda.lib().kda_chunk_fwd_workspace_size(B, T, H, 128, 128, 1)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device="cuda")
    out = {}
    out["fwd"] = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"])
    out["fwd_seg"] = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], workspace=ws)
    dO = torch.randn(B, T, H, 128, device="cuda", generator=torch.Generator(device="cuda").manual_seed(3))
    out["bwd"] = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], dO.to(torch.bfloat16))
    S = W.decode_state(W.DECODE_256x32, device="cuda", seed=72, N=4)
    tok = W.decode_tokens(W.DECODE_256x32, device="cuda", seed=72, N=4, steps=1)
    o = kda.recurrent_step(tok["q"][0], tok["k"][0], tok["v"][0], tok["g"][0], tok["beta"][0], S)
    out["dec"] = (o, S)
    torch.cuda.synchronize()
    return out


def _flat(x):
    if isinstance(x, dict):
        return [t for k in sorted(x) for t in _flat(x[k])]
    if isinstance(x, (tuple, list)):
        return [t for y in x for t in _flat(y)]
    return [] if x is None else [x]


def test_sync_debug_same_results(kda, monkeypatch):
    monkeypatch.delenv("KDA_SYNC_DEBUG", raising=False)
    ref = _calls(kda)
    monkeypatch.setenv("KDA_SYNC_DEBUG", "1")
    got = _calls(kda)
    for name in ref:
        for a, b in zip(_flat(ref[name]), _flat(got[name])):
            assert torch.equal(a, b), name
