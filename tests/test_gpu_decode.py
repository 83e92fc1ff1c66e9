"""GPU parity of the one-token decode step against the fp64 oracle, through
the C ABI.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import BF16_REL_L2, check_step, head_rel_l2, rms, to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_61_amd as kda
    kda.lib()
    return kda


def _check_step(o_g, o_r, dtype, what):
    return check_step(o_g, o_r, dtype, what)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("d", [64, 128])
def test_steps_small(kda, dtype, d):
    cfg = W.Decode("small", 5, 3, d, d, 12, dtype, 0.05)
    S = W.decode_state(cfg, device="cuda")
    tok = W.decode_tokens(cfg, device="cuda")
    S_ref = to64(S)
    for t in range(cfg.steps):
        args = [tok[n][t].contiguous() for n in ("q", "k", "v", "g", "beta")]
        o = kda.recurrent_step(*args, S)
        torch.cuda.synchronize()
        o_r, S_ref = oracle.recurrent_step(*[to64(a) for a in args], S_ref)
        _check_step(to64(o), o_r, dtype, f"step {t}")
    err = np.max(np.abs(to64(S) - S_ref))
    assert err <= 1e-5 * rms(S_ref), err


def test_decode_workload_256x32(kda):
    """The decode workload at full size (256 sequences x 32 heads, 64 steps):
    every head's o at every step and every head's final state against the
    oracle, which runs the same 64 steps on its own fp64 copy of the state."""
    cfg = W.DECODE_256x32
    S = W.decode_state(cfg, device="cuda")
    tok = W.decode_tokens(cfg, device="cuda")
    S_ref = to64(S)
    worst = {}
    for t in range(cfg.steps):
        args = [tok[n][t] for n in ("q", "k", "v", "g", "beta")]
        o = kda.recurrent_step(*args, S)
        o_r, S_ref = oracle.recurrent_step(*[to64(a) for a in args], S_ref, inplace=True)
        torch.cuda.synchronize()
        st = _check_step(to64(o), o_r, torch.bfloat16, f"step {t}")
        for key, val in st.items():
            worst[key] = max(worst.get(key, 0.0), val)
    rel_s = head_rel_l2(to64(S), S_ref, (0, 1))
    print(f"[parity] decode 256x32 x64: worst over steps " + " ".join(f"{k}={v:.3e}" for k, v in worst.items())
          + f"; final state per-head rel L2 {rel_s:.3e}", flush=True)
    assert rel_s <= BF16_REL_L2
    assert torch.isfinite(S).all()


def test_decode_matches_prefill(kda):
    """T decode steps and one prefill over the same tokens agree (both vs the
    oracle, and with each other within the bf16 bounds)."""
    cfg = W.PREFILL_BF16_H16_T4K
    inp = W.prefill_inputs(cfg, device="cuda", seed=8, B=2, T=70, H=3)
    o_p, S_p = kda.chunk_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"])
    S = inp["S0"].clone()
    outs = []
    for t in range(70):
        outs.append(kda.recurrent_step(*(inp[n][:, t].contiguous() for n in ("q", "k", "v", "g", "beta")), S))
    torch.cuda.synchronize()
    o_d = torch.stack(outs, 1)
    rel = (o_d.float() - o_p.float()).norm() / o_p.float().norm()
    assert rel < 5e-3
    assert ((S - S_p).norm() / S_p.norm()) < 5e-3


def test_zero_sequences_is_noop(kda):
    z = torch.empty((0, 4, 128), dtype=torch.bfloat16, device="cuda")
    S = torch.empty((0, 4, 128, 128), dtype=torch.float32, device="cuda")
    o = kda.recurrent_step(z, z, z, z, torch.empty((0, 4), dtype=torch.bfloat16, device="cuda"), S)
    assert o.shape == (0, 4, 128)
