"""Pins for the token-by-token fp64 oracle (CPU only).

Each test ties the oracle to something other than itself: a closed form, a
special case that reduces to a textbook result, a hand-worked example, an
explicit-matrix brute force, or an invariant the mathematics fixes.  Pages:
  [HLA-1] "Hybrid Linear Attention Architecture: Making LLM Training and Inference More Efficient"
  [HLA-4] "Demystifying Hybrid LLM Architectures: Linear Attention, Residuals, and Latent MoE"
  [HLA-5] "Linear Attention Architecture Deep Dive: From State Updates to Efficient Chunked Computation"
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
TOL = 1e-12


def _rand_case(rng, B=1, T=7, H=2, dk=5, dv=3, gate=True, s0=True):
    q = rng.standard_normal((B, T, H, dk))
    k = rng.standard_normal((B, T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, dv))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, H))))
    g = -np.log1p(np.exp(rng.standard_normal((B, T, H, dk)) - 1.0)) if gate else np.zeros((B, T, H, dk))
    S0 = rng.standard_normal((B, H, dk, dv)) if s0 else None
    return q, k, v, g, beta, S0


def _orthonormal(rng, n, d):
    """n orthonormal rows in R^d (n <= d), from the QR of a Gaussian."""
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    return Qm[:, :n].T.copy()


# ---------------------------------------------------------------- P1
def test_single_token_closed_form(rng):
    """[HLA-1] §3.3 KDA equation, one token, written as explicit matrices:
    S1 = (I - beta k k^T) Diag(exp g) S0 + beta k v^T, o = S1^T q."""
    dk, dv = 6, 4
    q, k, v, g, beta, S0 = _rand_case(rng, T=1, H=1, dk=dk, dv=dv)
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    kk, vv, qq, gg, bb = k[0, 0, 0], v[0, 0, 0], q[0, 0, 0], g[0, 0, 0], beta[0, 0, 0]
    S1 = (np.eye(dk) - bb * np.outer(kk, kk)) @ np.diag(np.exp(gg)) @ S0[0, 0] + bb * np.outer(kk, vv)
    assert np.max(np.abs(ST[0, 0] - S1)) < TOL
    assert np.max(np.abs(o[0, 0, 0] - S1.T @ qq)) < TOL
    # with S0 = 0 the state is the rank-one write and o = beta (k.q) v
    o0, ST0 = oracle.recurrent_fwd(q, k, v, g, beta, None)
    assert np.max(np.abs(ST0[0, 0] - bb * np.outer(kk, vv))) < TOL
    assert np.max(np.abs(o0[0, 0, 0] - bb * (kk @ qq) * vv)) < TOL


# ---------------------------------------------------------------- P2
def test_beta_zero_is_pure_decay(rng):
    """beta -> 0 means no update ([HLA-1] §3.2): only the gates act, so
    S_t = Diag(exp sum_{m<=t} g_m) S0 and o_t = S_t^T q_t."""
    q, k, v, g, beta, S0 = _rand_case(rng, T=9, H=2, dk=5, dv=3)
    beta = np.zeros_like(beta)
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    cum = np.cumsum(g, axis=1)                       # [B,T,H,dk]
    for h in range(2):
        for t in range(9):
            St = np.exp(cum[0, t, h])[:, None] * S0[0, h]
            assert np.max(np.abs(o[0, t, h] - St.T @ q[0, t, h])) < TOL
        assert np.max(np.abs(ST[0, h] - np.exp(cum[0, -1, h])[:, None] * S0[0, h])) < TOL
    # and with g = 0 as well, S is unchanged and o_t = S0^T q_t
    o2, ST2 = oracle.recurrent_fwd(q, k, v, np.zeros_like(g), beta, S0)
    assert np.max(np.abs(ST2 - S0)) < TOL
    assert np.max(np.abs(o2[0, :, 0] - q[0, :, 0] @ S0[0, 0])) < TOL


# ---------------------------------------------------------------- P3
def test_orthonormal_keys_reduce_to_causal_linear_attention(rng):
    """With orthonormal keys, beta = 1, g = 0 and S0 = 0 the erase term k^T S
    vanishes, so KDA is plain causal linear attention ([HLA-1] §3.1):
    O = Tril(Q K^T) V and S_T = K^T V."""
    T, dk, dv = 8, 8, 5
    K = _orthonormal(rng, T, dk)
    Q = rng.standard_normal((T, dk))
    V = rng.standard_normal((T, dv))
    q, k, v = Q[None, :, None], K[None, :, None], V[None, :, None]
    g = np.zeros((1, T, 1, dk))
    beta = np.ones((1, T, 1))
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, None)
    assert np.max(np.abs(o[0, :, 0] - np.tril(Q @ K.T) @ V)) < 1e-12
    assert np.max(np.abs(ST[0, 0] - K.T @ V)) < 1e-12


# ---------------------------------------------------------------- P4
@pytest.mark.parametrize("T", [3, 8])
def test_orthonormal_recall_and_flush(rng, T):
    """beta = 1 is a complete overwrite ([HLA-1] §3.2): with orthonormal keys
    and g = 0, S_T = (I - K^T K) S0 + K^T V, every key recalls its own value
    (S_T^T k_i = v_i), and after d_k orthogonal steps S0 is fully flushed."""
    dk, dv = 8, 4
    K = _orthonormal(rng, T, dk)
    V = rng.standard_normal((T, dv))
    S0 = rng.standard_normal((1, 1, dk, dv))
    q = rng.standard_normal((1, T, 1, dk))
    o, ST = oracle.recurrent_fwd(q, K[None, :, None], V[None, :, None],
                                 np.zeros((1, T, 1, dk)), np.ones((1, T, 1)), S0)
    S = ST[0, 0]
    assert np.max(np.abs(S - ((np.eye(dk) - K.T @ K) @ S0[0, 0] + K.T @ V))) < 1e-12
    assert np.max(np.abs(K @ S - V)) < 1e-12
    if T == dk:
        assert np.max(np.abs(S - K.T @ V)) < 1e-12


# ---------------------------------------------------------------- P5
def test_decay_first_worked_example():
    """Hand-worked example (tests/golden): decay before erase/write, [HLA-1] §3.3."""
    with open(os.path.join(GOLDEN, "decay_first_example.json")) as f:
        ex = json.load(f)
    inp, exp = ex["inputs"], ex["expected"]
    q = np.array(inp["q"])[None, None, None]
    k = np.array(inp["k"])[None, None, None]
    v = np.array(inp["v"])[None, None, None]
    g = np.array(inp["g"])[None, None, None]
    beta = np.array([[[inp["beta"]]]])
    S0 = np.array(inp["S0"])[None, None]
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    assert np.max(np.abs(ST[0, 0] - np.array(exp["S1"]))) < 1e-15
    assert np.max(np.abs(o[0, 0, 0] - np.array(exp["o"]))) < 1e-15


# ---------------------------------------------------------------- P7
def test_brute_force_transition_products(rng):
    """Explicit d_k x d_k transition matrices M_t = (I - beta k k^T) Diag(alpha)
    ([HLA-1] §3.3): S_t = (prod M) S0 + sum_j (prod_{i>j} M_i) beta_j k_j v_j^T,
    evaluated as matrix products, independent of the oracle's loop."""
    T, dk, dv = 6, 4, 3
    q, k, v, g, beta, S0 = _rand_case(rng, T=T, H=1, dk=dk, dv=dv)
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    M = [(np.eye(dk) - beta[0, t, 0] * np.outer(k[0, t, 0], k[0, t, 0])) @ np.diag(np.exp(g[0, t, 0]))
         for t in range(T)]
    for t in range(T):
        # prod_{i<=t} M_i applied to S0, newest on the left
        prod = np.eye(dk)
        for i in range(t + 1):
            prod = M[i] @ prod
        St = prod @ S0[0, 0]
        for j in range(t + 1):
            pj = np.eye(dk)
            for i in range(j + 1, t + 1):
                pj = M[i] @ pj
            St = St + pj @ (beta[0, j, 0] * np.outer(k[0, j, 0], v[0, j, 0]))
        assert np.max(np.abs(o[0, t, 0] - St.T @ q[0, t, 0])) < 1e-12
        if t == T - 1:
            assert np.max(np.abs(ST[0, 0] - St)) < 1e-12


# ---------------------------------------------------------------- P8
def test_split_invariance_and_decode_equals_prefill(rng):
    """Streaming carries only the state ([HLA-5] §5, §8.2): running [0,T1) then
    [T1,T) from the hand-off state equals one run, and T single-token decode
    steps equal the prefill."""
    B, T, H, dk, dv = 2, 11, 2, 5, 4
    q, k, v, g, beta, S0 = _rand_case(rng, B=B, T=T, H=H, dk=dk, dv=dv)
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    T1 = 4
    oa, Sa = oracle.recurrent_fwd(q[:, :T1], k[:, :T1], v[:, :T1], g[:, :T1], beta[:, :T1], S0)
    ob, Sb = oracle.recurrent_fwd(q[:, T1:], k[:, T1:], v[:, T1:], g[:, T1:], beta[:, T1:], Sa)
    assert np.max(np.abs(np.concatenate([oa, ob], axis=1) - o)) < TOL
    assert np.max(np.abs(Sb - ST)) < TOL
    S = S0.copy()
    for t in range(T):
        ot, S = oracle.recurrent_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        assert np.max(np.abs(ot - o[:, t])) < TOL
    assert np.max(np.abs(S - ST)) < TOL


def test_linearity_in_values_and_state(rng):
    """For fixed keys, gates and beta the map (V, S0) -> (O, S_T) is linear."""
    q, k, v1, g, beta, S01 = _rand_case(rng, T=6, H=1, dk=4, dv=3)
    v2 = rng.standard_normal(v1.shape)
    S02 = rng.standard_normal(S01.shape)
    a, b = 0.7, -1.3
    o1, s1 = oracle.recurrent_fwd(q, k, v1, g, beta, S01)
    o2, s2 = oracle.recurrent_fwd(q, k, v2, g, beta, S02)
    o3, s3 = oracle.recurrent_fwd(q, k, a * v1 + b * v2, g, beta, a * S01 + b * S02)
    assert np.max(np.abs(o3 - (a * o1 + b * o2))) < 1e-12
    assert np.max(np.abs(s3 - (a * s1 + b * s2))) < 1e-12


def test_scalar_gate_matches_gated_deltanet(rng):
    """A channel-constant gate is the scalar-gated rule of [HLA-1] §3.3,
    S_t = alpha_t (I - beta k k^T) S_{t-1} + beta v k^T (in d_k x d_v form)."""
    T, dk, dv = 5, 4, 3
    q, k, v, _, beta, S0 = _rand_case(rng, T=T, H=1, dk=dk, dv=dv)
    a = -np.abs(rng.standard_normal(T)) * 0.5
    g = np.repeat(a[None, :, None, None], dk, axis=3)
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    S = S0[0, 0].copy()
    for t in range(T):
        kk = k[0, t, 0]
        S = np.exp(a[t]) * (np.eye(dk) - beta[0, t, 0] * np.outer(kk, kk)) @ S + beta[0, t, 0] * np.outer(kk, v[0, t, 0])
        assert np.max(np.abs(o[0, t, 0] - S.T @ q[0, t, 0])) < 1e-12
    assert np.max(np.abs(ST[0, 0] - S)) < 1e-12


def test_delta_rule_ungated_matches_retrieve_erase_write(rng):
    """g = 0 is the delta rule; its "retrieve, erase, write" form of [HLA-4]
    §2.3 (S <- S + beta k (v - S^T k)^T, then y = S^T q) must agree."""
    T, dk, dv = 7, 5, 2
    q, k, v, _, beta, S0 = _rand_case(rng, T=T, H=1, dk=dk, dv=dv)
    o, ST = oracle.recurrent_fwd(q, k, v, np.zeros((1, T, 1, dk)), beta, S0)
    S = S0[0, 0].copy()
    for t in range(T):
        kk = k[0, t, 0]
        retrieved = S.T @ kk
        S = S + beta[0, t, 0] * np.outer(kk, v[0, t, 0] - retrieved)
        assert np.max(np.abs(o[0, t, 0] - S.T @ q[0, t, 0])) < 1e-12
    assert np.max(np.abs(ST[0, 0] - S)) < 1e-12


# ---------------------------------------------------------------- P9
def test_norm_growth_bound(rng):
    """With ||k|| = 1, beta in [0,1] and alpha <= 1 the transition is a
    contraction, so ||S_t||_F <= ||S_{t-1}||_F + beta_t ||v_t||."""
    T, dk, dv = 40, 6, 5
    q, k, v, g, beta, S0 = _rand_case(rng, T=T, H=1, dk=dk, dv=dv)
    S = S0[:, 0][:, None]
    for t in range(T):
        prev = np.linalg.norm(S)
        _, S = oracle.recurrent_step(q[:, t], k[:, t], v[:, t], g[:, t], beta[:, t], S)
        assert np.linalg.norm(S) <= prev + beta[0, t, 0] * np.linalg.norm(v[0, t, 0]) + 1e-12


# ---------------------------------------------------------------- P10
def test_full_overwrite_latest_value_wins(rng):
    """beta = 1 with the same unit key repeated: the latest value replaces the
    old one (S_t^T k = v_t): [HLA-1] §3.2 and [HLA-4] §2.3 give beta = 1 as a
    full overwrite."""
    T, dk, dv = 6, 5, 3
    kk = rng.standard_normal(dk)
    kk /= np.linalg.norm(kk)
    k = np.tile(kk, (1, T, 1, 1))
    v = rng.standard_normal((1, T, 1, dv))
    q = np.tile(kk, (1, T, 1, 1))            # read with the same key
    S0 = rng.standard_normal((1, 1, dk, dv))
    o, ST = oracle.recurrent_fwd(q, k, v, np.zeros((1, T, 1, dk)), np.ones((1, T, 1)), S0)
    assert np.max(np.abs(o[0, :, 0] - v[0, :, 0])) < 1e-12


def test_gate_clears_channel(rng):
    """A channel with alpha -> 0 is cleared before the write ([HLA-1] §3.3,
    "exponentially suppress old memories"): with beta = 0 and g_c = -50 the
    row of that channel falls by exp(-50)."""
    dk, dv = 4, 3
    q, k, v, g, beta, S0 = _rand_case(rng, T=1, H=1, dk=dk, dv=dv)
    g = np.zeros_like(g)
    g[0, 0, 0, 2] = -50.0
    _, ST = oracle.recurrent_fwd(q, k, v, g, np.zeros_like(beta), S0)
    assert np.max(np.abs(ST[0, 0, 2])) <= np.exp(-50) * np.max(np.abs(S0[0, 0, 2])) * (1 + 1e-12)
    assert np.max(np.abs(ST[0, 0, [0, 1, 3]] - S0[0, 0, [0, 1, 3]])) == 0.0


def test_empty_sequence_returns_initial_state(rng):
    q, k, v, g, beta, S0 = _rand_case(rng, T=0, H=2)
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, S0)
    assert o.shape[1] == 0
    assert np.array_equal(ST, S0)


# ------------------------------------------------- variants: scalar gate, no delta
def test_scalar_gate_mode_is_gated_deltanet(rng):
    """The scalar-gate mode (one log-gate per token and head) against the
    scalar-gated rule of [HLA-1] §3.3 written as explicit matrices,
    S_t = alpha_t (I - beta k k^T) S_{t-1} + beta k v^T (d_k x d_v form)."""
    T, dk, dv = 6, 4, 3
    q, k, v, _, beta, S0 = _rand_case(rng, T=T, H=2, dk=dk, dv=dv)
    a = -np.abs(rng.standard_normal((1, T, 2))) * 0.5
    o, ST = oracle.recurrent_fwd(q, k, v, a, beta, S0, scalar_gate=True)
    for h in range(2):
        S = S0[0, h].copy()
        for t in range(T):
            kk = k[0, t, h]
            S = np.exp(a[0, t, h]) * (np.eye(dk) - beta[0, t, h] * np.outer(kk, kk)) @ S \
                + beta[0, t, h] * np.outer(kk, v[0, t, h])
            assert np.max(np.abs(o[0, t, h] - S.T @ q[0, t, h])) < TOL
        assert np.max(np.abs(ST[0, h] - S)) < TOL


def test_no_delta_ungated_is_causal_linear_attention(rng):
    """Without the delta rule and with alpha = 1 the state is the plain sum of
    writes, S_t = S_0 + sum_{s<=t} k_s v_s^T ([HLA-1] §3.1), so the read-out is
    causal linear attention: o_t = S_0^T q_t + sum_{s<=t} (k_s . q_t) v_s."""
    T, dk, dv = 7, 5, 3
    q, k, v, _, _, S0 = _rand_case(rng, T=T, H=1, dk=dk, dv=dv)
    o, ST = oracle.recurrent_fwd(q, k, v, np.zeros((1, T, 1, dk)), None, S0, delta=False)
    for t in range(T):
        ref = S0[0, 0].T @ q[0, t, 0] + sum((k[0, s, 0] @ q[0, t, 0]) * v[0, s, 0] for s in range(t + 1))
        assert np.max(np.abs(o[0, t, 0] - ref)) < TOL
    assert np.max(np.abs(ST[0, 0] - (S0[0, 0] + np.einsum("sc,sj->cj", k[0, :, 0], v[0, :, 0])))) < TOL


def test_no_delta_gated_closed_form(rng):
    """Per-channel decay without the delta rule (GLA / RWKV-6 form of [HLA-1]
    §3.3): unrolling the recurrence, channel c of the state is
    prod_{r<=t} alpha_rc S0[c] + sum_{s<=t} k_sc v_s prod_{s<r<=t} alpha_rc;
    beta plays no part."""
    T, dk, dv = 6, 4, 3
    q, k, v, g, beta, S0 = _rand_case(rng, T=T, H=1, dk=dk, dv=dv)
    o, ST = oracle.recurrent_fwd(q, k, v, g, beta, S0, delta=False)
    o2, _ = oracle.recurrent_fwd(q, k, v, g, None, S0, delta=False)
    assert np.array_equal(o, o2)
    G = np.cumsum(g[0, :, 0], axis=0)          # G[t, c] = sum_{r<=t} g_rc
    for t in range(T):
        S = np.exp(G[t])[:, None] * S0[0, 0]
        for s in range(t + 1):
            S = S + np.exp(G[t] - G[s])[:, None] * np.outer(k[0, s, 0], v[0, s, 0])
        assert np.max(np.abs(o[0, t, 0] - S.T @ q[0, t, 0])) < TOL
        if t == T - 1:
            assert np.max(np.abs(ST[0, 0] - S)) < TOL


def test_variant_steps_equal_prefill(rng):
    """T decode steps equal one prefill of T tokens in every variant (the
    streaming consistency of [HLA-5] §5)."""
    T, dk, dv = 5, 4, 3
    q, k, v, g, beta, S0 = _rand_case(rng, T=T, H=2, dk=dk, dv=dv)
    for scalar_gate in (False, True):
        gg = g[..., 0] if scalar_gate else g
        for delta in (True, False):
            o, ST = oracle.recurrent_fwd(q, k, v, gg, beta, S0, scalar_gate=scalar_gate, delta=delta)
            S = S0.copy()                      # [N = 1, H, dk, dv]
            for t in range(T):
                ot, S = oracle.recurrent_step(q[:, t], k[:, t], v[:, t], gg[:, t], beta[:, t], S,
                                              scalar_gate=scalar_gate, delta=delta)
                assert np.max(np.abs(ot - o[:, t])) < TOL
            assert np.max(np.abs(S - ST)) < TOL
