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
 *     delta rule (Gated DeltaNet) of [HLA-1] §3.2, alpha_t times the identity.
 *   KDA_ORACLE_NO_DELTA: no erase step, S_t = Diag(alpha_t) S_{t-1} + k_t v_t^T
 *     -- per-channel decay without the delta rule (GLA / RWKV-6,
 *     [HLA-1] §3.3, first formula); beta is not used. */
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

/* Number of OpenMP threads a parallel region would use (for reporting). */
int kda_oracle_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}
