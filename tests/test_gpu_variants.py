"""GPU parity of the two variants of the recurrence against the fp64 oracle,
through the C ABI: the scalar forget gate (Gated DeltaNet, "Hybrid Linear
Attention Architecture: Making LLM Training and Inference More Efficient"
§3.3) and per-channel decay without the delta rule (GLA / RWKV-6, same page
§3.3), each alone and combined, in the chunked prefill (one pass and
segmented) and in the decode step.  Needs an MI355X and the built library."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import BF16_REL_L2, check_prefill, oracle_prefill, rms, to64
from tests.test_gpu_decode import _check_step

pytestmark = pytest.mark.gpu

# (scalar_gate, delta)
VARIANTS = [(True, True), (False, False), (True, False)]
VIDS = ["scalar", "nodelta", "scalar-nodelta"]


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_61_amd as kda
    kda.lib()
    return kda


def _case(B, T, H, seed, scalar_gate, s0=True, cfg=W.PREFILL_BF16_H16_T4K):
    inp = W.prefill_inputs(cfg, device="cuda", seed=seed, B=B, T=T, H=H, scalar_gate=scalar_gate)
    if not s0:
        inp["S0"] = None
    return inp


def _run(kda, inp, scalar_gate, delta, beta=True):
    o, S = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"] if beta else None, inp["S0"],
                         scalar_gate=scalar_gate, delta=delta)
    torch.cuda.synchronize()
    return o, S


SHAPES = [(1, 1, 2, True), (1, 63, 2, True), (1, 64, 1, False), (2, 130, 3, True), (1, 517, 2, True),
          (3, 192, 1, False)]


@pytest.mark.parametrize("B,T,H,s0", SHAPES, ids=[f"B{b}T{t}H{h}{'-S0' if z else ''}" for b, t, h, z in SHAPES])
@pytest.mark.parametrize("scalar_gate,delta", VARIANTS, ids=VIDS)
def test_prefill_small(kda, B, T, H, s0, scalar_gate, delta):
    """Single-chunk, exact, ragged and multi-chunk lengths, with and without S0."""
    inp = _case(B, T, H, 700 + T + 5 * H, scalar_gate, s0)
    print(f"case variant scalar_gate={scalar_gate} delta={delta} B{B} T{T} H{H} s0={s0}", flush=True)
    o, S = _run(kda, inp, scalar_gate, delta)
    o_ref, S_ref = oracle_prefill(inp, scalar_gate=scalar_gate, delta=delta)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"B{B}T{T}H{H}")


SEG = [(1, 64 * 13 + 17, 2, 4, True), (2, 64 * 20, 1, 5, False)]


@pytest.mark.parametrize("B,T,H,nseg,s0", SEG, ids=[f"B{b}T{t}H{h}-seg{n}" for b, t, h, n, _ in SEG])
@pytest.mark.parametrize("scalar_gate,delta", VARIANTS, ids=VIDS)
def test_prefill_segmented(kda, B, T, H, nseg, s0, scalar_gate, delta, monkeypatch):
    """The segmented schedule of each variant against the oracle and against
    the variant's one-pass schedule."""
    flags = (1 if scalar_gate else 0) | (0 if delta else 2)
    monkeypatch.setenv("KDA_SEGMENTS", str(nseg))
    assert kda.lib().kda_chunk_fwd_ex_workspace_size(B, T, H, 128, 128, 1, flags) > 0
    inp = _case(B, T, H, 900 + T + nseg, scalar_gate, s0)
    print(f"case variant segmented scalar_gate={scalar_gate} delta={delta} B{B} T{T} H{H} nseg={nseg}", flush=True)
    o, S = _run(kda, inp, scalar_gate, delta)
    o_ref, S_ref = oracle_prefill(inp, scalar_gate=scalar_gate, delta=delta)
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"segmented B{B}T{T}H{H}")
    monkeypatch.setenv("KDA_SEGMENTS", "0")
    assert kda.lib().kda_chunk_fwd_ex_workspace_size(B, T, H, 128, 128, 1, flags) == 0
    o1, S1 = _run(kda, inp, scalar_gate, delta)
    assert (o.float() - o1.float()).norm() / o1.float().norm() < 5e-3
    assert (S - S1).norm() / S1.norm() < 1e-3


@pytest.mark.parametrize("scalar_gate,delta", VARIANTS, ids=VIDS)
def test_prefill_B8_H32_T8192(kda, scalar_gate, delta):
    """The B8 H32 T8192 workload at full size in each variant (the launch the
    variant benchmark times), all 256 heads against the oracle."""
    cfg = W.PREFILL_BF16_B8_H32_T8K
    inp = W.prefill_inputs(cfg, device="cuda", scalar_gate=scalar_gate)
    print(f"case variant full B8 H32 T8192 scalar_gate={scalar_gate} delta={delta}", flush=True)
    o, S = _run(kda, inp, scalar_gate, delta)
    assert torch.isfinite(o.float()).all() and torch.isfinite(S).all()
    o_ref, S_ref = oracle_prefill(inp, scalar_gate=scalar_gate, delta=delta)
    del inp
    check_prefill(to64(o), to64(S), o_ref, S_ref, torch.bfloat16, f"variant B8 H32 T8192 sg={scalar_gate} d={delta}")


def test_no_delta_ignores_beta(kda):
    """Without the delta rule beta is not read: a NULL beta and a real one
    give identical results."""
    for scalar_gate in (False, True):
        inp = _case(1, 300, 2, 17, scalar_gate)
        o1, S1 = _run(kda, inp, scalar_gate, False, beta=True)
        o2, S2 = _run(kda, inp, scalar_gate, False, beta=False)
        assert torch.equal(o1, o2) and torch.equal(S1, S2)


def test_scalar_gate_equals_broadcast_gate(kda):
    """A scalar gate is the per-channel gate with every channel equal: the
    scalar-gate path against the KDA path fed the broadcast gate."""
    for delta in (True, False):
        inp = _case(2, 200, 3, 23, True)
        o1, S1 = _run(kda, inp, True, delta)
        full = dict(inp)
        full["g"] = inp["g"][..., None].expand(*inp["g"].shape, 128).contiguous()
        o2, S2 = _run(kda, full, False, delta)
        same = torch.equal(o1, o2) and torch.equal(S1, S2)
        print(f"delta={delta}: bit-identical={same}", flush=True)
        assert (o1.float() - o2.float()).norm() / o2.float().norm() < 1e-3
        assert (S1 - S2).norm() / S2.norm() < 1e-4


def test_variant_streaming_split(kda):
    """S_T may alias S0 in the variants too: [0,T1) then [T1,T) from the
    hand-off state equals the oracle on the whole sequence."""
    for scalar_gate, delta in VARIANTS:
        inp = _case(1, 300, 2, 29, scalar_gate)
        S = inp["S0"].clone()
        part = lambda t, a, b: t[:, a:b].contiguous()
        outs = []
        for a, b in ((0, 100), (100, 300)):
            o, _ = kda.chunk_fwd(*(part(inp[n], a, b) for n in ("q", "k", "v", "g", "beta")), S, S_T=S,
                                 scalar_gate=scalar_gate, delta=delta)
            outs.append(o)
        torch.cuda.synchronize()
        o_ref, S_ref = oracle_prefill(inp, scalar_gate=scalar_gate, delta=delta)
        check_prefill(to64(torch.cat(outs, 1)), to64(S), o_ref, S_ref, torch.bfloat16, "variant split")


@pytest.mark.parametrize("scalar_gate,delta", VARIANTS, ids=VIDS)
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "fp32"])
@pytest.mark.parametrize("d", [64, 128])
def test_decode_steps(kda, scalar_gate, delta, dtype, d):
    cfg = W.Decode("small", 5, 3, d, d, 12, dtype, 0.05)
    S = W.decode_state(cfg, device="cuda")
    tok = W.decode_tokens(cfg, device="cuda", scalar_gate=scalar_gate)
    S_ref = to64(S)
    for t in range(cfg.steps):
        q, k, v, g, beta = (tok[n][t].contiguous() for n in ("q", "k", "v", "g", "beta"))
        if not delta:
            beta = None
        o = kda.recurrent_step(q, k, v, g, beta, S, scalar_gate=scalar_gate, delta=delta)
        torch.cuda.synchronize()
        o_r, S_ref = oracle.recurrent_step(to64(q), to64(k), to64(v), to64(g), to64(beta), S_ref,
                                           scalar_gate=scalar_gate, delta=delta)
        _check_step(to64(o), o_r, dtype, f"step {t}")
    err = np.max(np.abs(to64(S) - S_ref))
    assert err <= 1e-5 * rms(S_ref), err


@pytest.mark.parametrize("scalar_gate,delta", VARIANTS, ids=VIDS)
def test_decode_matches_prefill(kda, scalar_gate, delta):
    """T decode steps of a variant and its prefill over the same tokens agree."""
    inp = _case(2, 70, 3, 31, scalar_gate)
    o_p, S_p = _run(kda, inp, scalar_gate, delta)
    S = inp["S0"].clone()
    outs = []
    for t in range(70):
        outs.append(kda.recurrent_step(*(inp[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")), S,
                                       scalar_gate=scalar_gate, delta=delta))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, 1)
    for b in range(2):
        for h in range(3):
            ref = o_d[b, :, h].float()
            assert (o_p[b, :, h].float() - ref).norm() / ref.norm() < 2 * BF16_REL_L2
    assert (S_p - S).norm() / S.norm() < 1e-3
