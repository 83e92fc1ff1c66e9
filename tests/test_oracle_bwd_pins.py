"""Pins for the backward oracle (CPU only).

The pages give no backward formulas; the gradient is fixed by the forward
definition alone.  The fp64 reverse-mode oracle (``oracle.recurrent_bwd``) is
pinned against
  * central finite differences of the forward oracle along random directions,
    for every input, every variant, with and without a final-state adjoint;
  * an independent fp64 implementation of the token recurrence written here in
    plain PyTorch CPU ops and differentiated by torch.autograd;
  * the composition rule for the per-chunk state adjoints: the adjoint of the
    state entering chunk n equals the dS0 of the backward run on the tokens
    from chunk n onwards, started from that state.
"""
import numpy as np
import pytest
import torch

import oracle

MODES = [(False, True), (True, True), (False, False), (True, False)]
MIDS = ["kda", "scalar", "nodelta", "scalar-nodelta"]


def _case(rng, B=2, T=11, H=2, dk=5, dv=3, scalar_gate=False):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    g = -np.abs(rng.standard_normal((B, T, H) if scalar_gate else (B, T, H, dk))) * 0.4
    beta = rng.uniform(0.05, 1.0, (B, T, H))
    S0 = rng.standard_normal((B, H, dk, dv))
    dO = rng.standard_normal((B, T, H, dv))
    dST = rng.standard_normal((B, H, dk, dv))
    return dict(q=q, k=k, v=v, g=g, beta=beta, S0=S0), dO, dST


def _loss(inp, dO, dST, scalar_gate, delta):
    o, ST = oracle.recurrent_fwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"] if delta else None,
                                 inp["S0"], scalar_gate=scalar_gate, delta=delta)
    val = float((o * dO).sum())
    if dST is not None:
        val += float((ST * dST).sum())
    return val


GRAD = dict(q="dq", k="dk", v="dv", g="dg", beta="dbeta", S0="dS0")


@pytest.mark.parametrize("scalar_gate,delta", MODES, ids=MIDS)
@pytest.mark.parametrize("with_dST", [True, False], ids=["dST", "no-dST"])
def test_finite_differences(scalar_gate, delta, with_dST):
    rng = np.random.default_rng(11 + 2 * scalar_gate + delta)
    inp, dO, dST = _case(rng, scalar_gate=scalar_gate)
    if not with_dST:
        dST = None
    gr = oracle.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"] if delta else None, inp["S0"],
                              dO, dST, scalar_gate=scalar_gate, delta=delta, chunk=4)
    eps = 1e-6
    for name, key in GRAD.items():
        if name == "beta" and not delta:
            assert np.all(gr[key] == 0.0)
            continue
        for _ in range(2):
            u = rng.standard_normal(inp[name].shape)
            xp = dict(inp); xp[name] = inp[name] + eps * u
            xm = dict(inp); xm[name] = inp[name] - eps * u
            fd = (_loss(xp, dO, dST, scalar_gate, delta) - _loss(xm, dO, dST, scalar_gate, delta)) / (2 * eps)
            an = float((gr[key] * u).sum())
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(fd)), (name, fd, an)


def _torch_forward(q, k, v, g, beta, S0, scalar_gate, delta):
    """The recurrence written independently with torch CPU ops (S is d_k x d_v,
    decay first, then erase / write, read after write)."""
    B, T, H, dk = q.shape
    outs = []
    S = S0.clone()
    for t in range(T):
        a = torch.exp(g[:, t])                      # [B,H] or [B,H,dk]
        a = a[..., None, None] if scalar_gate else a[..., None]
        S = a * S
        kt, vt = k[:, t], v[:, t]
        if delta:
            r = torch.einsum("bhc,bhcj->bhj", kt, S)
            S = S + beta[:, t][..., None, None] * kt[..., :, None] * (vt - r)[..., None, :]
        else:
            S = S + kt[..., :, None] * vt[..., None, :]
        outs.append(torch.einsum("bhc,bhcj->bhj", q[:, t], S))
    return torch.stack(outs, 1), S


@pytest.mark.parametrize("scalar_gate,delta", MODES, ids=MIDS)
def test_matches_torch_autograd(scalar_gate, delta):
    rng = np.random.default_rng(23 + 2 * scalar_gate + delta)
    inp, dO, dST = _case(rng, B=2, T=13, H=2, dk=6, dv=4, scalar_gate=scalar_gate)
    ts = {n: torch.tensor(x, dtype=torch.float64, requires_grad=True) for n, x in inp.items()}
    o, ST = _torch_forward(ts["q"], ts["k"], ts["v"], ts["g"], ts["beta"], ts["S0"], scalar_gate, delta)
    loss = (o * torch.tensor(dO)).sum() + (ST * torch.tensor(dST)).sum()
    names = [n for n in GRAD if delta or n != "beta"]
    grads = torch.autograd.grad(loss, [ts[n] for n in names])
    gr = oracle.recurrent_bwd(inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"] if delta else None, inp["S0"],
                              dO, dST, scalar_gate=scalar_gate, delta=delta, chunk=5)
    for n, gt in zip(names, grads):
        ref = gt.numpy()
        assert np.max(np.abs(gr[GRAD[n]] - ref)) <= 1e-10 * max(1.0, np.max(np.abs(ref))), n


@pytest.mark.parametrize("chunk", [1, 3, 4, 64])
def test_chunk_length_only_changes_recomputation(chunk):
    """The checkpoint block length is an implementation detail: every result
    is the same to rounding."""
    rng = np.random.default_rng(5)
    inp, dO, dST = _case(rng, T=17)
    ref = oracle.recurrent_bwd(*(inp[n] for n in ("q", "k", "v", "g", "beta", "S0")), dO, dST, chunk=17)
    gr = oracle.recurrent_bwd(*(inp[n] for n in ("q", "k", "v", "g", "beta", "S0")), dO, dST, chunk=chunk)
    for key in GRAD.values():
        assert np.max(np.abs(gr[key] - ref[key])) <= 1e-12 * max(1.0, np.max(np.abs(ref[key]))), key


def test_chunk_adjoints_compose():
    """dS_chunks[n] (adjoint of the state entering chunk n) equals dS0 of the
    backward over tokens [n*C, T) started from the forward state at n*C; and
    dS_chunks[0] equals dS0."""
    rng = np.random.default_rng(7)
    C = 4
    inp, dO, dST = _case(rng, B=1, T=14, H=2)
    gr = oracle.recurrent_bwd(*(inp[n] for n in ("q", "k", "v", "g", "beta", "S0")), dO, dST, chunk=C,
                              chunk_adjoints=True)
    assert gr["dS_chunks"].shape == (1, 2, 4, 5, 3)
    assert np.array_equal(gr["dS_chunks"][:, :, 0], gr["dS0"])
    for n in (1, 2, 3):
        t0 = n * C
        _, S_t0 = oracle.recurrent_fwd(*(inp[x][:, :t0] for x in ("q", "k", "v", "g", "beta")), inp["S0"])
        tail = oracle.recurrent_bwd(*(inp[x][:, t0:] for x in ("q", "k", "v", "g", "beta")), S_t0,
                                    dO[:, t0:], dST, chunk=C)
        assert np.max(np.abs(tail["dS0"] - gr["dS_chunks"][:, :, n])) <= 1e-12 * max(1.0, np.abs(tail["dS0"]).max())


def test_output_adjoint_only_reaches_earlier_tokens():
    """Causality: the adjoint of o_t changes no gradient of a later token."""
    rng = np.random.default_rng(9)
    inp, dO, _ = _case(rng, B=1, T=10, H=1)
    dO[:, 6:] = 0.0
    gr = oracle.recurrent_bwd(*(inp[n] for n in ("q", "k", "v", "g", "beta", "S0")), dO, None)
    for key in ("dq", "dk", "dv", "dg", "dbeta"):
        assert np.all(gr[key][:, 6:] == 0.0), key


def test_scalar_gate_gradient_is_the_channel_sum():
    """A scalar gate is the per-channel gate with all channels equal; by the
    chain rule through that broadcast, its gradient is the channel sum of the
    per-channel gradient (the GPU path computes it that way)."""
    rng = np.random.default_rng(31)
    inp, dO, dST = _case(rng, B=2, T=9, H=2, dk=5, dv=3, scalar_gate=True)
    sc = oracle.recurrent_bwd(*(inp[n] for n in ("q", "k", "v", "g", "beta", "S0")), dO, dST, scalar_gate=True)
    gfull = np.repeat(inp["g"][..., None], 5, axis=-1)
    per = oracle.recurrent_bwd(inp["q"], inp["k"], inp["v"], gfull, inp["beta"], inp["S0"], dO, dST)
    assert np.max(np.abs(per["dg"].sum(-1) - sc["dg"])) <= 1e-12 * max(1.0, np.abs(sc["dg"]).max())
    for key in ("dq", "dk", "dv", "dbeta", "dS0"):
        assert np.max(np.abs(per[key] - sc[key])) <= 1e-12 * max(1.0, np.abs(sc[key]).max()), key
