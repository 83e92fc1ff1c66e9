"""Chunkwise-parallel KDA in NumPy fp64 -- TEST INFRASTRUCTURE ONLY.

This is the hardware-efficient chunkwise form that the pages give for the
gated delta rule ("Hybrid Linear Attention Architecture: Making LLM Training
and Inference More Efficient" §IV; "Hybrid Linear Attention Architecture:
Technical Deep Dive and Implementation Guide" §4; "Linear Attention
Architecture Deep Dive: From State Updates to Efficient Chunked Computation"
§5), taken step by step in the pages' notation, with library primitives
(matmul, a unit-triangular solve) as steps and no further blocking or fusion.
It exists to expose the per-chunk intermediates that the GPU stages produce,
and it is pinned to the token-by-token definition (it must equal it for every
chunk length, including C = 1, where it collapses to the recurrence).

Readings of the pages taken here (the printed chunk equations are garbled):

* The gate factor that multiplies queries and keys inside a chunk is the
  prefix product up to and including position i, Gamma_i = exp(b_i) with
  b_i = sum_{m<=i} g_m (the in-chunk cumulative log-gate of §IV's "accumulating
  gate products in log-space").  Keys are divided by it (K / Gamma).
* The factor that carries a key to the chunk end in the state update is the
  suffix product Gamma^{i->C} = exp(b_C - b_i), exclusive of i.
* gamma^C = exp(b_C), the whole-chunk decay.
* U and W (left undefined on the pages beyond "value representations") are
  U = A Diag(beta) V and W = A Diag(beta) (Gamma * K) with
  A = (I + StrictTril(Diag(beta) (Gamma*K) (K/Gamma)^T))^{-1}; then U - W S is
  the residual correction of §IV ("predict, then write the residual").
* Tril in the output keeps the diagonal: a token reads its own write.
These are the only placements for which the chunked and token forms agree;
the agreement is what the tests check.
"""
from __future__ import annotations

import numpy as np
from scipy.linalg import solve_triangular


def chunk_fwd(q, k, v, g, beta, S0=None, C: int = 64, keep: bool = False):
    """Chunked forward.  Shapes as in ``oracle.recurrent_fwd``.

    Returns (o, S_T) or, with keep=True, (o, S_T, inter) where inter holds
      'b'     [B,T,H,dk]  in-chunk inclusive cumulative log-gate
      'W','U' [B,T,H,dk] / [B,T,H,dv]
      'Delta' [B,T,H,dv]  U - W S_[t]
      'S'     [B,H,N,dk,dv] chunk-entry states S_[t]
    """
    q, k, v, g, beta = (np.asarray(a, dtype=np.float64) for a in (q, k, v, g, beta))
    B, T, H, dk = q.shape
    dv = v.shape[-1]
    N = (T + C - 1) // C
    o = np.zeros((B, T, H, dv))
    ST = np.zeros((B, H, dk, dv))
    if keep:
        inter = {"b": np.zeros((B, T, H, dk)), "W": np.zeros((B, T, H, dk)),
                 "U": np.zeros((B, T, H, dv)), "Delta": np.zeros((B, T, H, dv)),
                 "S": np.zeros((B, H, N, dk, dv))}
    for bb in range(B):
        for h in range(H):
            S = np.zeros((dk, dv)) if S0 is None else np.array(S0[bb, h], dtype=np.float64)
            for n in range(N):
                s, e = n * C, min(T, (n + 1) * C)
                Q, K, V = q[bb, s:e, h], k[bb, s:e, h], v[bb, s:e, h]
                G, beta_c = g[bb, s:e, h], beta[bb, s:e, h]
                Lc = e - s
                # cumulative log-gates inside the chunk (log space)
                bcum = np.cumsum(G, axis=0)                 # b_i, inclusive
                Gam = np.exp(bcum)                          # Gamma^{1->i}
                gam_C = np.exp(bcum[-1])                    # gamma^C
                Gam_iC = np.exp(bcum[-1][None, :] - bcum)   # Gamma^{i->C}, exclusive of i
                Qg, Kg, Kd = Q * Gam, K * Gam, K / Gam      # Gamma*Q, Gamma*K, K/Gamma
                # UT transform: A = (I + L)^{-1}, W, U
                L = np.tril(beta_c[:, None] * (Kg @ Kd.T), -1)
                I = np.eye(Lc)
                W = solve_triangular(I + L, beta_c[:, None] * Kg, lower=True, unit_diagonal=True)
                U = solve_triangular(I + L, beta_c[:, None] * V, lower=True, unit_diagonal=True)
                # residual correction and output
                Delta = U - W @ S
                O = Qg @ S + np.tril(Qg @ Kd.T) @ Delta
                if keep:
                    inter["b"][bb, s:e, h] = bcum
                    inter["W"][bb, s:e, h] = W
                    inter["U"][bb, s:e, h] = U
                    inter["Delta"][bb, s:e, h] = Delta
                    inter["S"][bb, h, n] = S
                o[bb, s:e, h] = O
                # inter-chunk state passing
                S = gam_C[:, None] * S + (Gam_iC * K).T @ Delta
            ST[bb, h] = S
    if keep:
        return o, ST, inter
    return o, ST
