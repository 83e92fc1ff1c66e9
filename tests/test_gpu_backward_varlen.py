"""GPU parity of the packed variable-length backward (kda_chunk_bwd_varlen)
against the fp64 reverse-mode oracle run on each sequence alone: each packed
sequence is an independent recurrence from its own entry state ("Linear
Attention Architecture Deep Dive: From State Updates to Efficient Chunked
Computation" §5), so its gradients are those of that sequence as a batch of
one.  Bounds as for the batched backward.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import to64
from tests.test_gpu_backward import NAMES, _check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_61_amd as kda
    kda.lib()
    return kda


def _packed(lengths, H, seed, scalar_gate=False, s0=True, dst=True):
    Tt = int(sum(lengths))
    inp = W.prefill_inputs(W.PREFILL_BF16_H16_T4K, device="cuda", seed=seed, B=1, T=max(Tt, 1), H=H,
                           scalar_gate=scalar_gate)
    x = {n: inp[n][0, :Tt].contiguous() for n in ("q", "k", "v", "g", "beta")}
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 1)
    N = len(lengths)
    x["S0"] = (torch.randn(N, H, 128, 128, device="cuda", generator=gen) * 0.02) if s0 else None
    x["dO"] = torch.randn(Tt, H, 128, device="cuda", generator=gen).to(torch.bfloat16)
    x["dST"] = (torch.randn(N, H, 128, 128, device="cuda", generator=gen) * 0.1) if dst else None
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    x["cu"] = torch.tensor(cu, dtype=torch.int32, device="cuda")
    return x, cu


def _run(kda, x, scalar_gate=False, delta=True):
    gr = kda.chunk_bwd_varlen(x["q"], x["k"], x["v"], x["g"], x["beta"] if delta else None, x["cu"], x["S0"],
                              x["dO"], x["dST"], scalar_gate=scalar_gate, delta=delta)
    torch.cuda.synchronize()
    return gr


def _check_seq(x, gr, i, a, b, scalar_gate, delta, what):
    sl = lambda t: to64(t[a:b])[None]
    one = lambda t: None if t is None else to64(t[i])[None]
    if b == a:
        want = torch.zeros_like(gr["dS0"][i]) if x["dST"] is None else x["dST"][i]
        assert torch.equal(gr["dS0"][i], want), f"{what}: empty sequence {i} must pass dS_T through"
        return
    g64 = sl(x["g"])
    ref = oracle.recurrent_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), g64, sl(x["beta"]) if delta else None,
                               one(x["S0"]), sl(x["dO"]), one(x["dST"]), scalar_gate=scalar_gate, delta=delta)
    got = {n: (to64(gr[n][i])[None] if n == "dS0" else sl(gr[n])) for n in NAMES if gr[n] is not None}
    scale = None
    if scalar_gate:
        # dg against sum_c |dg_c| of the per-channel gradient on the broadcast gate
        gfull = np.repeat(g64[..., None], 128, axis=-1)
        per = oracle.recurrent_bwd(sl(x["q"]), sl(x["k"]), sl(x["v"]), gfull, sl(x["beta"]) if delta else None,
                                   one(x["S0"]), sl(x["dO"]), one(x["dST"]), delta=delta)["dg"]
        scale = np.abs(per).sum(-1)
    _check(got, ref, f"{what} seq {i} T={b - a}", dg_scale=scale)


MIX = [1, 63, 0, 64, 65, 200, 130]


def test_mixed_lengths(kda):
    x, cu = _packed(MIX, 2, 61)
    print(f"case bwd varlen {MIX} H2", flush=True)
    gr = _run(kda, x)
    for i in range(len(MIX)):
        _check_seq(x, gr, i, int(cu[i]), int(cu[i + 1]), False, True, "varlen")


@pytest.mark.parametrize("scalar_gate,delta", [(True, True), (False, False), (True, False)],
                         ids=["scalar", "nodelta", "scalar-nodelta"])
def test_mixed_lengths_variants(kda, scalar_gate, delta):
    lengths = [70, 0, 129, 5]
    x, cu = _packed(lengths, 2, 71 + 2 * scalar_gate + delta, scalar_gate=scalar_gate, dst=False)
    print(f"case bwd varlen {lengths} H2 scalar_gate={scalar_gate} delta={delta}", flush=True)
    gr = _run(kda, x, scalar_gate, delta)
    for i in range(len(lengths)):
        _check_seq(x, gr, i, int(cu[i]), int(cu[i + 1]), scalar_gate, delta, "varlen variant")


def test_matches_batched_backward(kda):
    """Equal lengths packed: the same gradients as the batched entry point
    (same kernels, different chunk-slot layout), bit for bit."""
    B, T, H = 3, 130, 2
    x, cu = _packed([T] * B, H, 81)
    gr = _run(kda, x)
    view = lambda t: t.view(B, T, *t.shape[1:])
    ref = kda.chunk_bwd(view(x["q"]), view(x["k"]), view(x["v"]), view(x["g"]), view(x["beta"]), x["S0"],
                        view(x["dO"]), x["dST"])
    torch.cuda.synchronize()
    for n in NAMES:
        got = gr[n] if n == "dS0" else view(gr[n])
        assert torch.equal(got, ref[n]), n


@pytest.mark.parametrize("scalar_gate,delta", [(False, True), (False, False), (True, True)],
                         ids=["kda", "nodelta", "scalar"])
def test_states_saved_packed(kda, scalar_gate, delta):
    """kda_chunk_fwd_varlen_save gives the outputs of the one-pass packed
    forward, and the packed backward on its workspace (KDA_STATES_SAVED) the
    gradients of the backward with its own state pass, bit for bit."""
    lengths = [130, 1, 64, 200, 7]
    x, cu = _packed(lengths, 3, 97, scalar_gate=scalar_gate)
    beta = x["beta"] if delta else None
    print(f"case varlen fwd_save + bwd scalar_gate={scalar_gate} delta={delta}", flush=True)
    kw = dict(scalar_gate=scalar_gate, delta=delta)
    o1, S1 = kda.chunk_fwd_varlen(x["q"], x["k"], x["v"], x["g"], beta, x["cu"], x["S0"], segmented=False, **kw)
    o2, S2, ws = kda.chunk_fwd_varlen_save(x["q"], x["k"], x["v"], x["g"], beta, x["cu"], x["S0"], **kw)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(S1, S2)
    g1 = kda.chunk_bwd_varlen(x["q"], x["k"], x["v"], x["g"], beta, x["cu"], x["S0"], x["dO"], x["dST"], **kw)
    g2 = kda.chunk_bwd_varlen(x["q"], x["k"], x["v"], x["g"], beta, x["cu"], x["S0"], x["dO"], x["dST"], **kw,
                              workspace=ws, states_saved=True)
    torch.cuda.synchronize()
    for n in g1:
        if g1[n] is not None:
            assert torch.equal(g1[n], g2[n]), n


def test_many_sequences(kda):
    """A serving mix: sequences of 1 .. 2048 tokens, 8 heads; every sequence
    against the oracle, all outputs finite."""
    lengths = W.packed_lengths(24000, 300.0, 9, max_len=2048)
    x, cu = _packed(lengths, 8, 91, dst=False)
    print(f"case bwd varlen {len(lengths)} sequences, T_total={cu[-1]}", flush=True)
    gr = _run(kda, x)
    for i in range(len(lengths)):
        _check_seq(x, gr, i, int(cu[i]), int(cu[i + 1]), False, True, "varlen many")
    for n in ("dq", "dk", "dv", "dg", "dbeta", "dS0"):
        assert torch.isfinite(gr[n].float()).all(), n
