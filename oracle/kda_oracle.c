/*
 * kda_oracle.c -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, fp64 CPU implementation of the KDA recurrence (gated delta rule
 * with a per-channel forget gate), token by token.  Only the test suite, the
 * smoke check and the CPU-baseline leg of the benchmark may load this file's
 * library; the product path never does.  It shares no code with the HIP path.
 *
 * Sources (page titles as published):
 *   [HLA-1] "Hybrid Linear Attention Architecture: Making LLM Training and
 *            Inference More Efficient"
 *   [HLA-4] "Demystifying Hybrid LLM Architectures: Linear Attention,
 *            Residuals, and Latent MoE"
 *
 * The update is the KDA rule of [HLA-1] §3.3 (last equation):
 *     S_t = (I - beta_t k_t k_t^T) Diag(alpha_t) S_{t-1} + beta_t k_t v_t^T
 * written with the state as a d_k x d_v matrix (row index = key channel), the
 * transpose of the pages' d_v x d_k picture, which the pages themselves say is
 * a matter of convention ([HLA-1] §III, opening paragraph).  [HLA-1] §3.3
 * states the order: the old state is first decayed per channel, then the
 * delta rule erases and writes.  The erase/write step is the "retrieve, erase,
 * write" loop of [HLA-1] §3.2 and [HLA-4] §2.3, and the read-out y_t = S_t q_t
 * follows the update ([HLA-4] §2.3 pseudocode, §2.1 retrieval), here
 * o_t = S_t^T q_t.  alpha_t = exp(g_t) with g_t the log-gate.
 *
 * Layouts (all row-major, contiguous, fp64):
 *   q, k, g : [B, T, H, dk]     v : [B, T, H, dv]     beta : [B, T, H]
 *   S0, ST  : [B, H, dk, dv]    o : [B, T, H, dv]
 * S0 == NULL means a zero initial state; ST == NULL means "do not write".
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#include <stdint.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Variants (flags of the _ex entry points):
 *   KDA_ORACLE_SCALAR_GATE: one log-gate per token and head, g [B, T, H]
 *     ([N, H] for a step), applied to every key channel -- the scalar-gated
 *     delta rule (Gated DeltaNet) of [HLA-1] §3.3 (its first formula), alpha_t times the identity.
 *   KDA_ORACLE_NO_DELTA: no erase step, S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T
 *     -- per-channel decay without the delta rule (GLA / RWKV-6,
 *     [HLA-1] §3.3, the element-wise gate); beta is not used. */
#define KDA_ORACLE_SCALAR_GATE 1
#define KDA_ORACLE_NO_DELTA 2

/* One token of the recurrence on one head's state S (dk x dv, fp64). */
static void kda_token(double *S, const double *q, const double *k,
                      const double *v, const double *g, double beta,
                      double *o, double *r, int64_t dk, int64_t dv, int flags)
{
    /* 1. per-channel forget gate: S <- Diag(exp g) S   ([HLA-1] §3.3) */
    for (int64_t c = 0; c < dk; ++c) {
        const double a = exp((flags & KDA_ORACLE_SCALAR_GATE) ? g[0] : g[c]);
        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] *= a;
    }
    if (flags & KDA_ORACLE_NO_DELTA) {
        /* write only: S <- S + k v^T                       ([HLA-1] §3.1) */
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j) S[c * dv + j] += k[c] * v[j];
    } else {
        /* 2. retrieve the value stored under k: r = S^T k   ([HLA-1] §3.2) */
        for (int64_t j = 0; j < dv; ++j) r[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j) r[j] += k[c] * S[c * dv + j];
        /* 3. erase and write: S <- S + beta k (v - r)^T
         *    (= (I - beta k k^T) S + beta k v^T)                ([HLA-1] §3.2) */
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j)
                S[c * dv + j] += beta * k[c] * (v[j] - r[j]);
    }
    /* 4. read after write: o = S^T q                      ([HLA-4] §2.3) */
    for (int64_t j = 0; j < dv; ++j) o[j] = 0.0;
    for (int64_t c = 0; c < dk; ++c)
        for (int64_t j = 0; j < dv; ++j) o[j] += q[c] * S[c * dv + j];
}

/* Full-sequence forward over T tokens for every (b, h) sequence.
 * Returns 0, or -1 on a bad argument / allocation failure. */
int kda_oracle_fwd_ex(const double *q, const double *k, const double *v,
                      const double *g, const double *beta, const double *S0,
                      double *o, double *ST, int64_t B, int64_t T, int64_t H,
                      int64_t dk, int64_t dv, int flags, int nthreads)
{
    if (!q || !k || !v || !g || !o) return -1;
    if (!beta && !(flags & KDA_ORACLE_NO_DELTA)) return -1;
    const int64_t gs = (flags & KDA_ORACLE_SCALAR_GATE) ? 1 : dk;   /* gate values per token */
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic, 1) reduction(| : failed)
#endif
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        double *S = (double *)malloc(sizeof(double) * (size_t)(dk * dv));
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!S || !r) { free(S); free(r); failed = 1; continue; }
        if (S0) memcpy(S, S0 + bh * dk * dv, sizeof(double) * (size_t)(dk * dv));
        else    memset(S, 0, sizeof(double) * (size_t)(dk * dv));
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = (b * T + t) * H + h;     /* index of (b,t,h) */
            kda_token(S, q + tok * dk, k + tok * dk, v + tok * dv,
                      g + tok * gs, beta ? beta[tok] : 0.0, o + tok * dv, r, dk, dv, flags);
        }
        if (ST) memcpy(ST + bh * dk * dv, S, sizeof(double) * (size_t)(dk * dv));
        free(S); free(r);
    }
    return failed ? -1 : 0;
}

int kda_oracle_fwd(const double *q, const double *k, const double *v,
                   const double *g, const double *beta, const double *S0,
                   double *o, double *ST, int64_t B, int64_t T, int64_t H,
                   int64_t dk, int64_t dv, int nthreads)
{
    return kda_oracle_fwd_ex(q, k, v, g, beta, S0, o, ST, B, T, H, dk, dv, 0, nthreads);
}

/* One decode step for N independent sequences: S [N,H,dk,dv] updated in
 * place, q,k,g [N,H,dk] (g [N,H] with a scalar gate), v [N,H,dv],
 * beta [N,H], o [N,H,dv]. */
int kda_oracle_step_ex(const double *q, const double *k, const double *v,
                       const double *g, const double *beta, double *S,
                       double *o, int64_t N, int64_t H, int64_t dk, int64_t dv,
                       int flags, int nthreads)
{
    if (!q || !k || !v || !g || !S || !o) return -1;
    if (!beta && !(flags & KDA_ORACLE_NO_DELTA)) return -1;
    const int64_t gs = (flags & KDA_ORACLE_SCALAR_GATE) ? 1 : dk;
    if (N < 0 || H < 0 || dk <= 0 || dv <= 0) return -1;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static) reduction(| : failed)
#endif
    for (int64_t nh = 0; nh < N * H; ++nh) {
        double *r = (double *)malloc(sizeof(double) * (size_t)dv);
        if (!r) { failed = 1; continue; }
        kda_token(S + nh * dk * dv, q + nh * dk, k + nh * dk, v + nh * dv,
                  g + nh * gs, beta ? beta[nh] : 0.0, o + nh * dv, r, dk, dv, flags);
        free(r);
    }
    return failed ? -1 : 0;
}

int kda_oracle_step(const double *q, const double *k, const double *v,
                    const double *g, const double *beta, double *S,
                    double *o, int64_t N, int64_t H, int64_t dk, int64_t dv,
                    int nthreads)
{
    return kda_oracle_step_ex(q, k, v, g, beta, S, o, N, H, dk, dv, 0, nthreads);
}

/* ------------------------------------------------------------------------
 * Backward: the derivative of the full-sequence forward above, by reverse-mode
 * differentiation of its token loop (chain rule through the same four steps
 * taken backwards).  Given the output adjoint dO [B,T,H,dv] and the adjoint
 * of the final state dST [B,H,dk,dv] (NULL: zero), it returns dq, dk, dv
 * [B,T,H,*], dg [B,T,H,dk] ([B,T,H] with a scalar gate), dbeta [B,T,H]
 * (zeros without the delta rule; may be NULL then) and dS0 [B,H,dk,dv]
 * (NULL: not written).  dSc, if not NULL, receives [B,H,ceil(T/chunk),dk,dv]:
 * entry n is the adjoint of the state at the start of token n*chunk (entry 0
 * equals dS0).
 *
 * For token t, with S_prev the state before it and D = Diag(exp g_t):
 *   forward:  Sd = D S_prev;  r = Sd^T k;  delta = beta (v - r);
 *             S = Sd + k delta^T;  o = S^T q
 *   backward (dS = adjoint of S, carried from token t+1):
 *             dS += q dO_t^T;         dq = S dO_t
 *             ddelta = dS^T k;        dk = dS delta;      dSd = dS
 *             dbeta = ddelta . (v - r);  dv = beta ddelta;  dr = -beta ddelta
 *             dSd += k dr^T;          dk += Sd dr
 *             dg_c = sum_j dSd[c][j] Sd[c][j];   dS <- D dSd
 * Without the delta rule S = Sd + k v^T, so dk = dS v, dv = dS^T k, dSd = dS.
 * The states of each block of `chunk` tokens are recomputed from a stored
 * block-entry state (memory: ceil(T/chunk) + chunk states per sequence).
 * ------------------------------------------------------------------------ */
static void kda_token_fwd_parts(const double *Sp, double *Sd, double *S, const double *k,
                                const double *v, const double *g, double beta,
                                double *r, double *delta, int64_t dk, int64_t dv, int flags)
{
    for (int64_t c = 0; c < dk; ++c) {
        const double a = exp((flags & KDA_ORACLE_SCALAR_GATE) ? g[0] : g[c]);
        for (int64_t j = 0; j < dv; ++j) Sd[c * dv + j] = a * Sp[c * dv + j];
    }
    if (flags & KDA_ORACLE_NO_DELTA) {
        for (int64_t j = 0; j < dv; ++j) { r[j] = 0.0; delta[j] = v[j]; }
    } else {
        for (int64_t j = 0; j < dv; ++j) r[j] = 0.0;
        for (int64_t c = 0; c < dk; ++c)
            for (int64_t j = 0; j < dv; ++j) r[j] += k[c] * Sd[c * dv + j];
        for (int64_t j = 0; j < dv; ++j) delta[j] = beta * (v[j] - r[j]);
    }
    for (int64_t c = 0; c < dk; ++c)
        for (int64_t j = 0; j < dv; ++j) S[c * dv + j] = Sd[c * dv + j] + k[c] * delta[j];
}

int kda_oracle_bwd_ex(const double *q, const double *k, const double *v,
                      const double *g, const double *beta, const double *S0,
                      const double *dO, const double *dST,
                      double *dq, double *dk_, double *dv_, double *dg, double *dbeta,
                      double *dS0, double *dSc, int64_t B, int64_t T, int64_t H,
                      int64_t dk, int64_t dv, int64_t chunk, int flags, int nthreads)
{
    if (!q || !k || !v || !g || !dO || !dq || !dk_ || !dv_ || !dg) return -1;
    const int nodelta = (flags & KDA_ORACLE_NO_DELTA) != 0;
    if (!nodelta && (!beta || !dbeta)) return -1;
    if (B < 0 || T < 0 || H < 0 || dk <= 0 || dv <= 0 || chunk <= 0) return -1;
    const int64_t gs = (flags & KDA_ORACLE_SCALAR_GATE) ? 1 : dk;
    const int64_t nblk = (T + chunk - 1) / chunk;
    const int64_t SZ = dk * dv;
    int failed = 0;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(dynamic) reduction(| : failed)
#endif
    for (int64_t bh = 0; bh < B * H; ++bh) {
        const int64_t b = bh / H, h = bh % H;
        double *ck = (double *)malloc(sizeof(double) * (size_t)((nblk + 1) * SZ));
        double *Sb = (double *)malloc(sizeof(double) * (size_t)((chunk + 1) * SZ));
        double *Sd = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *S = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *dS = (double *)malloc(sizeof(double) * (size_t)SZ);
        double *w = (double *)malloc(sizeof(double) * (size_t)(4 * dv + 2 * dk));
        if (!ck || !Sb || !Sd || !S || !dS || !w) {
            failed = 1;
            free(ck); free(Sb); free(Sd); free(S); free(dS); free(w);
            continue;
        }
        double *r = w, *delta = w + dv, *ddelta = w + 2 * dv, *dr = w + 3 * dv;
        /* forward: block-entry states */
        if (S0) memcpy(ck, S0 + bh * SZ, sizeof(double) * (size_t)SZ);
        else memset(ck, 0, sizeof(double) * (size_t)SZ);
        for (int64_t t = 0; t < T; ++t) {
            const int64_t tok = (b * T + t) * H + h;
            const double *Sp = ck + (t / chunk) * SZ;
            double *Sn = ck + (t / chunk) * SZ + ((t + 1) % chunk == 0 ? SZ : 0);
            /* within a block the running state lives in S; it is copied to the
             * next block's entry at the block end */
            kda_token_fwd_parts(t % chunk == 0 ? Sp : S, Sd, S, k + tok * dk, v + tok * dv,
                                g + tok * gs, beta ? beta[tok] : 0.0, r, delta, dk, dv, flags);
            if ((t + 1) % chunk == 0) memcpy(Sn, S, sizeof(double) * (size_t)SZ);
        }
        /* backward */
        if (dST) memcpy(dS, dST + bh * SZ, sizeof(double) * (size_t)SZ);
        else memset(dS, 0, sizeof(double) * (size_t)SZ);
        for (int64_t blk = nblk - 1; blk >= 0; --blk) {
            const int64_t t0 = blk * chunk, t1 = (t0 + chunk < T) ? t0 + chunk : T;
            /* Sb[i] = state before token t0 + i */
            memcpy(Sb, ck + blk * SZ, sizeof(double) * (size_t)SZ);
            for (int64_t t = t0; t < t1 - 1; ++t) {
                const int64_t tok = (b * T + t) * H + h;
                kda_token_fwd_parts(Sb + (t - t0) * SZ, Sd, Sb + (t - t0 + 1) * SZ, k + tok * dk,
                                    v + tok * dv, g + tok * gs, beta ? beta[tok] : 0.0, r, delta, dk, dv,
                                    flags);
            }
            for (int64_t t = t1 - 1; t >= t0; --t) {
                const int64_t tok = (b * T + t) * H + h;
                const double *qt = q + tok * dk, *kt = k + tok * dk, *vt = v + tok * dv;
                const double *gt = g + tok * gs, *dot = dO + tok * dv;
                const double bt = beta ? beta[tok] : 0.0;
                kda_token_fwd_parts(Sb + (t - t0) * SZ, Sd, S, kt, vt, gt, bt, r, delta, dk, dv, flags);
                /* o = S^T q */
                for (int64_t c = 0; c < dk; ++c) {
                    double acc = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        dS[c * dv + j] += qt[c] * dot[j];
                        acc += S[c * dv + j] * dot[j];
                    }
                    dq[tok * dk + c] = acc;
                }
                double *dkt = dk_ + tok * dk, *dvt = dv_ + tok * dv;
                if (nodelta) {
                    /* S = Sd + k v^T */
                    for (int64_t c = 0; c < dk; ++c) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < dv; ++j) acc += dS[c * dv + j] * vt[j];
                        dkt[c] = acc;
                    }
                    for (int64_t j = 0; j < dv; ++j) {
                        double acc = 0.0;
                        for (int64_t c = 0; c < dk; ++c) acc += dS[c * dv + j] * kt[c];
                        dvt[j] = acc;
                    }
                    if (dbeta) dbeta[tok] = 0.0;
                } else {
                    /* S = Sd + k delta^T */
                    for (int64_t j = 0; j < dv; ++j) {
                        double acc = 0.0;
                        for (int64_t c = 0; c < dk; ++c) acc += dS[c * dv + j] * kt[c];
                        ddelta[j] = acc;
                    }
                    for (int64_t c = 0; c < dk; ++c) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < dv; ++j) acc += dS[c * dv + j] * delta[j];
                        dkt[c] = acc;
                    }
                    /* delta = beta (v - r) */
                    double db = 0.0;
                    for (int64_t j = 0; j < dv; ++j) {
                        db += ddelta[j] * (vt[j] - r[j]);
                        dvt[j] = bt * ddelta[j];
                        dr[j] = -bt * ddelta[j];
                    }
                    dbeta[tok] = db;
                    /* r = Sd^T k: dSd += k dr^T, dk += Sd dr (dS now holds dSd) */
                    for (int64_t c = 0; c < dk; ++c) {
                        double acc = 0.0;
                        for (int64_t j = 0; j < dv; ++j) {
                            acc += Sd[c * dv + j] * dr[j];
                            dS[c * dv + j] += kt[c] * dr[j];
                        }
                        dkt[c] += acc;
                    }
                }
                /* Sd = D S_prev */
                if (flags & KDA_ORACLE_SCALAR_GATE) {
                    double acc = 0.0;
                    for (int64_t i = 0; i < SZ; ++i) acc += dS[i] * Sd[i];
                    dg[tok] = acc;
                    const double a = exp(gt[0]);
                    for (int64_t i = 0; i < SZ; ++i) dS[i] *= a;
                } else {
                    for (int64_t c = 0; c < dk; ++c) {
                        const double a = exp(gt[c]);
                        double acc = 0.0;
                        for (int64_t j = 0; j < dv; ++j) {
                            acc += dS[c * dv + j] * Sd[c * dv + j];
                            dS[c * dv + j] *= a;
                        }
                        dg[tok * dk + c] = acc;
                    }
                }
                if (dSc && t % chunk == 0)
                    memcpy(dSc + (bh * nblk + t / chunk) * SZ, dS, sizeof(double) * (size_t)SZ);
            }
        }
        if (dS0) memcpy(dS0 + bh * SZ, dS, sizeof(double) * (size_t)SZ);
        free(ck); free(Sb); free(Sd); free(S); free(dS); free(w);
    }
    return failed ? -1 : 0;
}

/* Number of OpenMP threads a parallel region would use (for reporting). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
