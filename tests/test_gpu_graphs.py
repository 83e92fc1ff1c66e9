"""The entry points run under HIP graph capture: a captured run of decode
steps and a captured prefill (one pass and segmented), replayed several times
with eager work and synchronisations in between, give bit-for-bit the eager
results on every replay.  Nothing in these paths allocates, synchronises or
records a memset.  Needs an MI355X."""
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


def _capture(fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def test_decode_steps_in_a_graph(kda):
    cfg = W.Decode("graph", 16, 4, 128, 128, 8, torch.bfloat16, 0.05)
    S0 = W.decode_state(cfg, device="cuda")
    tok = W.decode_tokens(cfg, device="cuda")
    steps = [[tok[n][t].contiguous() for n in ("q", "k", "v", "g", "beta")] for t in range(cfg.steps)]
    # eager reference
    S_ref = S0.clone()
    o_ref = [kda.recurrent_step(*steps[t], S_ref) for t in range(cfg.steps)]
    torch.cuda.synchronize()
    # captured
    S = S0.clone()
    outs = [torch.empty(cfg.N, cfg.H, 128, dtype=torch.bfloat16, device="cuda") for _ in range(cfg.steps)]

    def run():
        for t in range(cfg.steps):
            kda.recurrent_step(*steps[t], S, o=outs[t])

    graph = _capture(run)
    for rep in range(3):
        S.copy_(S0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t in range(cfg.steps):
            assert torch.equal(outs[t], o_ref[t]), (rep, t)
        assert torch.equal(S, S_ref), rep
        _ = (S0 * 2).sum().item()   # unrelated eager work between replays


@pytest.mark.parametrize("nseg", ["0", "4"], ids=["one-pass", "segmented"])
def test_prefill_in_a_graph(kda, nseg, monkeypatch):
    monkeypatch.setenv("KDA_SEGMENTS", nseg)
    inp = W.prefill_inputs(W.PREFILL_BF16_H16_T4K, device="cuda", seed=3, B=1, T=64 * 13 + 5, H=4)
    o_ref, S_ref = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"])
    torch.cuda.synchronize()
    o = torch.empty_like(o_ref)
    S_T = torch.empty_like(S_ref)
    wsz = kda.lib().kda_chunk_fwd_workspace_size(1, inp["q"].shape[1], 4, 128, 128, 1)
    assert (wsz > 0) == (nseg != "0")
    ws = torch.empty(max(wsz, 1), dtype=torch.uint8, device="cuda")

    def run():
        kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], o=o, S_T=S_T, workspace=ws)

    graph = _capture(run)
    for rep in range(3):
        o.zero_()
        S_T.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), rep
        assert torch.equal(S_T, S_ref), rep
