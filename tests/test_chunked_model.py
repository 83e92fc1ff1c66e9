"""Pins for the chunkwise fp64 model (CPU only).

The chunked form is stated to be mathematically equivalent to the recurrence
("Demystifying Hybrid LLM Architectures: Linear Attention, Residuals, and
Latent MoE" §2.4) and chunking must not change results ("Linear Attention
Architecture Deep Dive: From State Updates to Efficient Chunked Computation"
§8.2), so the model must equal the token oracle for every chunk length,
including a ragged last chunk, and at C = 1 it collapses to the recurrence.
"""
import numpy as np
import pytest

import oracle
from oracle import chunked


def _case(rng, B, T, H, dk, dv, mu=-3.0, s0=True):
    q = rng.standard_normal((B, T, H, dk)); q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k = rng.standard_normal((B, T, H, dk)); k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = 1 / (1 + np.exp(-rng.standard_normal((B, T, H))))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H, dk)) + mu))
    S0 = rng.standard_normal((B, H, dk, dv)) * 0.1 if s0 else None
    return q, k, v, g, beta, S0


@pytest.mark.parametrize("C", [1, 2, 16, 64])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_chunked_equals_recurrence(rng, C, T):
    q, k, v, g, beta, S0 = _case(rng, 1, T, 2, 8, 6)
    o_r, S_r = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    o_c, S_c = chunked.chunk_fwd(q, k, v, g, beta, S0, C=C)
    scale = max(1.0, np.max(np.abs(o_r)))
    assert np.max(np.abs(o_c - o_r)) < 1e-11 * scale
    assert np.max(np.abs(S_c - S_r)) < 1e-11 * max(1.0, np.max(np.abs(S_r)))


def test_chunked_full_width_heads(rng):
    """d_k = d_v = 128, C = 64, two chunks plus a ragged tail, strong gates."""
    q, k, v, g, beta, S0 = _case(rng, 1, 150, 1, 128, 128, mu=-1.0)
    o_r, S_r = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    o_c, S_c = chunked.chunk_fwd(q, k, v, g, beta, S0, C=64)
    assert np.max(np.abs(o_c - o_r)) < 1e-10
    assert np.max(np.abs(S_c - S_r)) < 1e-10


def test_intermediates_are_consistent(rng):
    """The exposed intermediates satisfy their defining relations:
    b is the in-chunk inclusive cumsum of g; Delta = U - W S_[t]; the chunk
    entry state of chunk n is the recurrence's state after n*C tokens."""
    C = 16
    q, k, v, g, beta, S0 = _case(rng, 1, 40, 1, 8, 4)
    o, ST, it = chunked.chunk_fwd(q, k, v, g, beta, S0, C=C, keep=True)
    for n in range(3):
        s, e = n * C, min(40, (n + 1) * C)
        assert np.allclose(it["b"][0, s:e, 0], np.cumsum(g[0, s:e, 0], axis=0), atol=1e-14)
        Delta = it["U"][0, s:e, 0] - it["W"][0, s:e, 0] @ it["S"][0, 0, n]
        assert np.allclose(Delta, it["Delta"][0, s:e, 0], atol=1e-13)
        if n == 0:
            assert np.allclose(it["S"][0, 0, 0], S0[0, 0])
        else:
            _, Sn = oracle.recurrent_fwd(q[:, :s], k[:, :s], v[:, :s], g[:, :s], beta[:, :s], S0)
            assert np.allclose(it["S"][0, 0, n], Sn[0, 0], atol=1e-12)


def test_unit_chunk_collapses_to_token_update(rng):
    """At C = 1: A = 1, W = beta Gamma k = beta exp(g) k, U = beta v."""
    q, k, v, g, beta, S0 = _case(rng, 1, 5, 1, 4, 3)
    _, _, it = chunked.chunk_fwd(q, k, v, g, beta, S0, C=1, keep=True)
    assert np.allclose(it["W"][0, :, 0], beta[0, :, 0, None] * np.exp(g[0, :, 0]) * k[0, :, 0], atol=1e-14)
    assert np.allclose(it["U"][0, :, 0], beta[0, :, 0, None] * v[0, :, 0], atol=1e-14)
