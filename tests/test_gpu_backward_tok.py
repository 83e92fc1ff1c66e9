"""GPU parity of the backward for fp32 inputs (d = 64 and 128) and bf16
inputs at d = 64 -- the token recurrence's reverse mode with chunk
checkpoints -- against the fp64 reverse-mode oracle, through the C ABI, for
KDA and its variants.  Needs an MI355X.

Tolerances: fp32 inputs and gradients: per-head relative L2 of every
gradient <= 1e-4 and max |err| <= 1e-3 RMS(reference) (the forward's fp32
bound is 1e-4 RMS on the max; a gradient is a longer chain of fp32 sums over
the sequence, so its max error gets ten times that).  bf16 at d = 64: the
bounds of the bf16 backward (per-head rel L2 <= 1e-2, max |err| beyond the
bf16 rounding of the reference <= 0.1 RMS)."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.parity import rms, rounding_floor, to64

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dg", "dbeta", "dS0")


@pytest.fixture(scope="module")
def kda():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gated_delta_rule_61_amd as kda
    kda.lib()
    return kda


def _inputs(dtype, d, B, T, H, seed, s0=True, dst=True, scalar_gate=False):
    cfg = W.Prefill("bwd_tok", B, T, H, d, d, dtype, 0.05 if s0 else None)
    inp = W.prefill_inputs(cfg, device="cuda", seed=seed, scalar_gate=scalar_gate)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed + 17)
    inp["dO"] = torch.randn(B, T, H, d, device="cuda", generator=gen).to(dtype)
    inp["dST"] = (torch.randn(B, H, d, d, device="cuda", generator=gen) * 0.1) if dst else None
    return inp


def _head_rel(g, r, axes):
    red = tuple(i for i in range(r.ndim) if i not in axes)
    num = np.sqrt(np.sum(np.square(g - r), axis=red))
    den = np.sqrt(np.sum(np.square(r), axis=red))
    ok = den > 0
    return float(np.max(num[ok] / den[ok])) if np.any(ok) else 0.0


def _case(kda, dtype, d, B, T, H, seed, s0=True, dst=True, scalar_gate=False, delta=True):
    inp = _inputs(dtype, d, B, T, H, seed, s0, dst, scalar_gate)
    what = f"{'fp32' if dtype == torch.float32 else 'bf16'} d{d} B{B} T{T} H{H} sg={scalar_gate} delta={delta}"
    print(f"case {what}", flush=True)
    gr = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"] if delta else None, inp["S0"],
                       inp["dO"], inp["dST"], scalar_gate=scalar_gate, delta=delta)
    torch.cuda.synchronize()
    x = [to64(inp[n]) for n in ("q", "k", "v", "g", "beta")]
    if not delta:
        x[4] = None
    ref = oracle.recurrent_bwd(*x, to64(inp["S0"]), to64(inp["dO"]), to64(inp["dST"]), scalar_gate=scalar_gate,
                               delta=delta)
    stats = {}
    for n in NAMES:
        if gr.get(n) is None or (n == "dbeta" and not delta):
            continue
        g, r = to64(gr[n]), ref[n]
        if r.size == 0:
            continue
        axes = (0, 1) if n == "dS0" else (0, 2)
        rel = _head_rel(g, r, axes)
        if dtype == torch.float32 or n == "dS0":
            mx = float(np.max(np.abs(g - r))) / max(rms(r), 1e-30)
        else:
            mx = float(np.max(np.abs(g - r) - rounding_floor(r))) / max(rms(r), 1e-30)
        stats[n] = (rel, mx)
    print(f"[bwd parity] {what}: " + " ".join(f"{n}=({a:.2e},{b:.2e})" for n, (a, b) in stats.items()), flush=True)
    rel_b, max_b = (1e-4, 1e-3) if dtype == torch.float32 else (1e-2, 0.1)
    for n, (a, b) in stats.items():
        if dtype != torch.float32 and n == "dS0":
            assert a <= rel_b and b <= 0.1, (what, n, a, b)
            continue
        assert a <= rel_b, f"{what}: {n} per-head rel L2 {a:.3e} > {rel_b}"
        assert b <= max_b, f"{what}: {n} max err {b:.3e} > {max_b} RMS"


SHAPES = [(1, 256, 2, False, False), (2, 65, 3, True, True), (1, 1, 1, True, True), (1, 200, 2, True, False),
          (1, 130, 1, False, True)]


@pytest.mark.parametrize("B,T,H,s0,dst", SHAPES, ids=[f"B{b}T{t}H{h}{'-S0' if s else ''}{'-dST' if d else ''}"
                                                     for b, t, h, s, d in SHAPES])
@pytest.mark.parametrize("d", [64, 128])
def test_fp32(kda, d, B, T, H, s0, dst):
    """fp32 at d = 64 (the fp32 workload's size, B1 H2 T256, first) and d = 128."""
    _case(kda, torch.float32, d, B, T, H, 2000 + T + H + d, s0, dst)


@pytest.mark.parametrize("scalar_gate,delta", [(True, True), (False, False), (True, False)],
                         ids=["scalar", "nodelta", "scalar-nodelta"])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16], ids=["fp32", "bf16"])
def test_variants_d64(kda, dtype, scalar_gate, delta):
    _case(kda, dtype, 64, 2, 150, 2, 3000, True, True, scalar_gate, delta)


@pytest.mark.parametrize("B,T,H", [(1, 300, 2), (2, 64, 3), (1, 1, 2)])
def test_bf16_d64(kda, B, T, H):
    _case(kda, torch.bfloat16, 64, B, T, H, 4000 + T + H)


def test_zero_length_fp32(kda):
    """T = 0: dS0 = dS_T, no token gradient."""
    inp = _inputs(torch.float32, 64, 2, 0, 3, 5)
    gr = kda.chunk_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"], inp["S0"], inp["dO"], inp["dST"])
    torch.cuda.synchronize()
    assert torch.equal(gr["dS0"], inp["dST"])
