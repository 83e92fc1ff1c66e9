"""Seeded synthetic workloads for the KDA prefill and decode paths.

This module only draws inputs; it holds none of the method's arithmetic, and
both the HIP path's tests/benchmark and the CPU oracle consume what it draws
(the oracle receives exact fp64 copies of the values the GPU receives).

Input recipe (per token and head):
  q, k  ~ N(0, 1), then L2-normalised over the channel axis (in fp32)
  v     ~ N(0, 1)
  beta  = sigmoid(N(0, 1))                      shape [B, T, H]
  g     = -softplus(N(mu, 1)), mu = -3 (or -5)  shape [B, T, H, d_k]   (log alpha)
  S0    = 0, or N(0, sigma) in fp32             shape [B, H, d_k, d_v]
then q, k, v, g, beta are cast to the workload's input dtype.  The second
argument of N(.,.) is a standard deviation.  For the scalar-gate variant g is
drawn the same way with one value per token and head (shape [B, T, H]); the
variant without the delta rule draws beta as usual and does not use it.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch
import torch.nn.functional as F


@dataclass(frozen=True)
class Prefill:
    name: str
    B: int
    T: int
    H: int
    dk: int
    dv: int
    dtype: torch.dtype
    s0_std: float | None     # None -> S0 = 0 (passed as a null pointer)
    gate_mu: float = -3.0
    seed: int = 0


@dataclass(frozen=True)
class Decode:
    name: str
    N: int
    H: int
    dk: int
    dv: int
    steps: int
    dtype: torch.dtype
    s_std: float
    gate_mu: float = -3.0
    seed: int = 4


# The five workloads of this path (index = position in the list).
PREFILL_FP32_SMALL = Prefill("kda_fwd_fp32_B1_H2_T256_d64", 1, 256, 2, 64, 64, torch.float32, None, -3.0, 0)
PREFILL_BF16_H16_T4K = Prefill("kda_fwd_bf16_B1_H16_T4096_d128", 1, 4096, 16, 128, 128, torch.bfloat16, 0.02, -3.0, 1)
PREFILL_BF16_B8_H32_T8K = Prefill("kda_fwd_bf16_B8_H32_T8192_d128", 8, 8192, 32, 128, 128, torch.bfloat16, None, -3.0, 2)
PREFILL_BF16_LONG_T128K = Prefill("kda_fwd_bf16_B1_H32_T131072_d128_slowgate", 1, 131072, 32, 128, 128, torch.bfloat16, None, -5.0, 3)
DECODE_256x32 = Decode("kda_decode_bf16_N256_H32_d128_x64", 256, 32, 128, 128, 64, torch.bfloat16, 0.05, -3.0, 4)

CONFIGS = [PREFILL_FP32_SMALL, PREFILL_BF16_H16_T4K, PREFILL_BF16_B8_H32_T8K,
           PREFILL_BF16_LONG_T128K, DECODE_256x32]


def _gen(device, seed: int) -> torch.Generator:
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    return gen


def _tokens(shape_lead, dk, dv, dtype, gate_mu, device, gen, scalar_gate=False):
    """Draw q, k, v, g, beta for a leading shape (e.g. (B,T,H) or (N,H))."""
    f32 = dict(dtype=torch.float32, device=device, generator=gen)
    q = torch.randn(*shape_lead, dk, **f32)
    k = torch.randn(*shape_lead, dk, **f32)
    v = torch.randn(*shape_lead, dv, **f32)
    beta = torch.sigmoid(torch.randn(*shape_lead, **f32))
    g = -F.softplus(torch.randn(*shape_lead, *(() if scalar_gate else (dk,)), **f32) + gate_mu)
    q = q / q.norm(dim=-1, keepdim=True)
    k = k / k.norm(dim=-1, keepdim=True)
    return [x.to(dtype).contiguous() for x in (q, k, v, g, beta)]


def prefill_inputs(cfg: Prefill, device="cpu", seed: int | None = None,
                   B: int | None = None, T: int | None = None, H: int | None = None,
                   scalar_gate: bool = False):
    """Return dict(q,k,v,g,beta,S0) for a prefill workload (shapes may be
    overridden to draw a smaller case with the same distributions)."""
    B = cfg.B if B is None else B
    T = cfg.T if T is None else T
    H = cfg.H if H is None else H
    gen = _gen(device, cfg.seed if seed is None else seed)
    q, k, v, g, beta = _tokens((B, T, H), cfg.dk, cfg.dv, cfg.dtype, cfg.gate_mu, device, gen, scalar_gate)
    S0 = None
    if cfg.s0_std is not None:
        S0 = (torch.randn(B, H, cfg.dk, cfg.dv, dtype=torch.float32, device=device,
                          generator=gen) * cfg.s0_std).contiguous()
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0)


def decode_state(cfg: Decode, device="cpu", seed: int | None = None, N: int | None = None):
    N = cfg.N if N is None else N
    gen = _gen(device, (cfg.seed if seed is None else seed) * 1000 + 7)
    return (torch.randn(N, cfg.H, cfg.dk, cfg.dv, dtype=torch.float32, device=device,
                        generator=gen) * cfg.s_std).contiguous()


def decode_tokens(cfg: Decode, device="cpu", seed: int | None = None, N: int | None = None,
                  steps: int | None = None, scalar_gate: bool = False):
    """Tokens for `steps` decode steps: dict of tensors with a leading step axis
    q,k,g [steps,N,H,dk], v [steps,N,H,dv], beta [steps,N,H]."""
    N = cfg.N if N is None else N
    steps = cfg.steps if steps is None else steps
    gen = _gen(device, cfg.seed if seed is None else seed)
    q, k, v, g, beta = _tokens((steps, N, cfg.H), cfg.dk, cfg.dv, cfg.dtype, cfg.gate_mu, device, gen,
                               scalar_gate)
    return dict(q=q, k=k, v=v, g=g, beta=beta)


def packed_lengths(total: int, mean: float, seed: int, max_len: int | None = None):
    """Sequence lengths for a packed batch: geometric with the given mean
    (a serving mix of many short and a few long requests), capped at max_len,
    drawn until they cover `total` tokens (the last one cut to fit)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    p = 1.0 / mean
    out, acc = [], 0
    while acc < total:
        u = float(torch.rand((), generator=gen))
        n = 1 + int(math.floor(math.log1p(-u) / math.log1p(-p))) if p < 1 else 1
        if max_len is not None:
            n = min(n, max_len)
        n = min(n, total - acc)
        out.append(n)
        acc += n
    return out
