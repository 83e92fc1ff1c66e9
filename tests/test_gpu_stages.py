"""Each step of the staged schedule against the fp64 chunked model's
intermediates (cumulative log-gates, W and U, the residual Delta and the
chunk-entry states, the output), through the C ABI.  Needs an MI355X."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import chunked
from tests.parity import to64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_61_amd as kda
    kda.lib()
    return kda


def _rel(a, b):
    n = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / n) if n > 0 else float(np.linalg.norm(a))


CASES = [(W.PREFILL_FP32_SMALL, 1, 150, 2, 1e-5), (W.PREFILL_BF16_H16_T4K, 1, 150, 2, 5e-3),
         (W.PREFILL_BF16_H16_T4K, 2, 64, 1, 5e-3)]


@pytest.mark.parametrize("cfg,B,T,H,tol", CASES, ids=[f"{c.dtype}-B{b}T{t}H{h}" for c, b, t, h, _ in CASES])
def test_each_stage(kda, cfg, B, T, H, tol):
    inp = W.prefill_inputs(cfg, device="cuda", seed=21, B=B, T=T, H=H)
    q, k, v, g, beta, S0 = (inp[n] for n in ("q", "k", "v", "g", "beta", "S0"))
    o_m, S_m, it = chunked.chunk_fwd(to64(q), to64(k), to64(v), to64(g), to64(beta), to64(S0), C=64, keep=True)

    b = kda.stage_cumsum(g)
    torch.cuda.synchronize()
    assert np.max(np.abs(to64(b) - it["b"])) <= 1e-5 * max(1.0, np.max(np.abs(it["b"])))

    # each later stage is fed the model's own (exact) inputs where it can be,
    # so that a mismatch points at that stage
    bm = torch.tensor(it["b"], dtype=torch.float32, device="cuda")
    Wg, Ug = kda.stage_ut(k, v, beta, bm)
    torch.cuda.synchronize()
    assert _rel(to64(Wg), it["W"]) <= tol, _rel(to64(Wg), it["W"])
    assert _rel(to64(Ug), it["U"]) <= tol, _rel(to64(Ug), it["U"])

    Wm = torch.tensor(it["W"], dtype=torch.float32, device="cuda")
    Um = torch.tensor(it["U"], dtype=torch.float32, device="cuda")
    Dg, Sc, ST = kda.stage_state(k, bm, Wm, Um, S0)
    torch.cuda.synchronize()
    assert _rel(to64(Dg), it["Delta"]) <= tol, _rel(to64(Dg), it["Delta"])
    assert _rel(to64(Sc), it["S"]) <= tol
    assert _rel(to64(ST), S_m) <= tol

    Dm = torch.tensor(it["Delta"], dtype=torch.float32, device="cuda")
    Sm = torch.tensor(it["S"], dtype=torch.float32, device="cuda")
    og = kda.stage_output(q, k, bm, Dm, Sm)
    torch.cuda.synchronize()
    assert _rel(to64(og), o_m) <= tol, _rel(to64(og), o_m)
