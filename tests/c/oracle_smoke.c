/* The fp64 oracle driven from C on small random cases, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer: every entry point and
 * variant runs, the forward agrees with T decode steps, and the backward's
 * adjoint at the start of the first chunk is dS0.  Exit status 0 on success.
 * Links oracle/kda_oracle.c (test infrastructure). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int kda_oracle_fwd_ex(const double*, const double*, const double*, const double*, const double*,
                      const double*, double*, double*, int64_t, int64_t, int64_t, int64_t, int64_t, int, int);
int kda_oracle_step_ex(const double*, const double*, const double*, const double*, const double*, double*,
                       double*, int64_t, int64_t, int64_t, int64_t, int, int);
int kda_oracle_bwd_ex(const double*, const double*, const double*, const double*, const double*, const double*,
                      const double*, const double*, double*, double*, double*, double*, double*, double*,
                      double*, int64_t, int64_t, int64_t, int64_t, int64_t, int64_t, int, int);

static uint64_t rs = 88172645463325252ull;
static double urand(void) {   /* xorshift64, uniform in (-1, 1) */
  rs ^= rs << 13; rs ^= rs >> 7; rs ^= rs << 17;
  return (double)(rs >> 11) / 4503599627370496.0 - 1.0;
}
static double* arr(int64_t n, double scale, double shift) {
  double* a = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  for (int64_t i = 0; i < n; ++i) a[i] = shift + scale * urand();
  return a;
}

int main(void) {
  const int64_t B = 2, T = 70, H = 3, dk = 8, dv = 5;
  for (int flags = 0; flags < 4; ++flags) {
    const int64_t gs = (flags & 1) ? 1 : dk;
    double *q = arr(B * T * H * dk, 0.5, 0), *k = arr(B * T * H * dk, 0.35, 0), *v = arr(B * T * H * dv, 1, 0);
    double *g = arr(B * T * H * gs, 0.05, -0.1), *beta = arr(B * T * H, 0.5, 0.5), *S0 = arr(B * H * dk * dv, 0.2, 0);
    double *o = arr(B * T * H * dv, 0, 0), *ST = arr(B * H * dk * dv, 0, 0);
    const double* bt = (flags & 2) ? NULL : beta;
    if (kda_oracle_fwd_ex(q, k, v, g, bt, S0, o, ST, B, T, H, dk, dv, flags, 2) != 0) return 1;
    /* T decode steps from S0 */
    double* S = arr(B * H * dk * dv, 0, 0);
    memcpy(S, S0, sizeof(double) * (size_t)(B * H * dk * dv));
    double *qs = arr(B * H * dk, 0, 0), *ks = arr(B * H * dk, 0, 0), *vs = arr(B * H * dv, 0, 0);
    double *gg = arr(B * H * gs, 0, 0), *bs = arr(B * H, 0, 0), *os = arr(B * H * dv, 0, 0);
    double err = 0;
    for (int64_t t = 0; t < T; ++t) {
      for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h) {
          const int64_t tok = (b * T + t) * H + h, n = b * H + h;
          memcpy(qs + n * dk, q + tok * dk, sizeof(double) * (size_t)dk);
          memcpy(ks + n * dk, k + tok * dk, sizeof(double) * (size_t)dk);
          memcpy(vs + n * dv, v + tok * dv, sizeof(double) * (size_t)dv);
          memcpy(gg + n * gs, g + tok * gs, sizeof(double) * (size_t)gs);
          bs[n] = beta[tok];
        }
      if (kda_oracle_step_ex(qs, ks, vs, gg, (flags & 2) ? NULL : bs, S, os, B, H, dk, dv, flags, 2) != 0) return 2;
      for (int64_t b = 0; b < B; ++b)
        for (int64_t h = 0; h < H; ++h)
          for (int64_t j = 0; j < dv; ++j)
            err = fmax(err, fabs(os[(b * H + h) * dv + j] - o[((b * T + t) * H + h) * dv + j]));
    }
    for (int64_t i = 0; i < B * H * dk * dv; ++i) err = fmax(err, fabs(S[i] - ST[i]));
    if (!(err < 1e-12)) { fprintf(stderr, "flags %d: forward vs steps %g\n", flags, err); return 3; }
    /* backward with per-chunk adjoints (chunk 16) */
    const int64_t nblk = (T + 15) / 16;
    double *dO = arr(B * T * H * dv, 1, 0), *dST = arr(B * H * dk * dv, 0.1, 0);
    double *dq = arr(B * T * H * dk, 0, 0), *dkk = arr(B * T * H * dk, 0, 0), *dvv = arr(B * T * H * dv, 0, 0);
    double *dg = arr(B * T * H * gs, 0, 0), *db = arr(B * T * H, 0, 0), *dS0 = arr(B * H * dk * dv, 0, 0);
    double* dSc = arr(B * H * nblk * dk * dv, 0, 0);
    if (kda_oracle_bwd_ex(q, k, v, g, bt, S0, dO, dST, dq, dkk, dvv, dg, db, dS0, dSc, B, T, H, dk, dv, 16, flags,
                          2) != 0)
      return 4;
    /* the adjoint of the state at the start of chunk 0 is dS0 */
    double e2 = 0;
    for (int64_t bh = 0; bh < B * H; ++bh)
      for (int64_t i = 0; i < dk * dv; ++i) e2 = fmax(e2, fabs(dSc[bh * nblk * dk * dv + i] - dS0[bh * dk * dv + i]));
    if (!(e2 < 1e-12)) { fprintf(stderr, "flags %d: chunk-0 adjoint vs dS0 %g\n", flags, e2); return 5; }
    free(q); free(k); free(v); free(g); free(beta); free(S0); free(o); free(ST); free(S);
    free(qs); free(ks); free(vs); free(gg); free(bs); free(os);
    free(dO); free(dST); free(dq); free(dkk); free(dvv); free(dg); free(db); free(dS0); free(dSc);
  }
  /* argument checks */
  if (kda_oracle_fwd_ex(NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 1, 1, 1, 1, 1, 0, 1) != -1) return 6;
  printf("oracle C smoke ok\n");
  return 0;
}
