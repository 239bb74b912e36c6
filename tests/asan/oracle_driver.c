/*
 * Host sanitizer driver for the float64 oracle (test infrastructure).  Built
 * with -fsanitize=address,undefined together with oracle/la_oracle.c by
 * tests/test_oracle_asan.py and run as a plain executable.  Every buffer is
 * allocated at exactly the size its routine reads or writes, so a read or
 * write past any of them stops the run; each routine is called on empty,
 * single-token and ragged shapes, with and without its optional arguments,
 * in both feature modes.  Two checks keep the calls honest: every output is
 * finite, and with constant rows of V the causal and non-causal outputs equal
 * that row (the weights of eq. 9 are positive and sum to one).
 */
#include <math.h>
#include <stdio.h>
#include <stdlib.h>

void orc_forward_causal(const double *, const double *, const double *, const double *, const double *, double *,
                        double *, double *, double *, long, long, long, long, long, long);
void orc_forward_causal_parallel(const double *, const double *, const double *, double *, double *, long, long,
                                 long, long, long);
void orc_forward_noncausal(const double *, const double *, const double *, double *, long, long, long, long, long,
                           long);
void orc_backward_causal(const double *, const double *, const double *, const double *, const double *,
                         const double *, const double *, const double *, double *, double *, double *, double *,
                         double *, long, long, long, long, long, long);
void orc_backward_noncausal(const double *, const double *, const double *, const double *, double *, double *,
                            double *, long, long, long, long, long, long);
void orc_forward_decay(const double *, const double *, const double *, const double *, const double *,
                       const double *, double *, double *, double *, double *, long, long, long, long, long, long);
void orc_backward_decay(const double *, const double *, const double *, const double *, const double *,
                        const double *, const double *, const double *, const double *, double *, double *, double *,
                        double *, double *, double *, long, long, long, long, long, long);
void orc_decode_step(const double *, const double *, const double *, const double *, double *, double *, double *,
                     long, long, long, long, long);
void orc_feature_performer(const double *, const double *, double *, long, long, long, long, long);
void orc_feature_performer_vjp(const double *, const double *, const double *, double *, long, long, long, long,
                               long);
void orc_feature_poly2(const double *, double *, long, long, long);
void orc_feature_poly2_vjp(const double *, const double *, double *, long, long, long);

static unsigned long long rng = 88172645463325252ull;
static double unif(void) { /* xorshift64, uniform in [-1, 1) */
  rng ^= rng << 13;
  rng ^= rng >> 7;
  rng ^= rng << 17;
  return (double)(rng >> 11) * (2.0 / 9007199254740992.0) - 1.0;
}
static int failures = 0;

/* exactly n doubles (at least one byte so that malloc returns a real block) */
static double *arr(long n, int fill) {
  double *p = (double *)malloc(n > 0 ? (size_t)n * sizeof(double) : 1);
  for (long i = 0; i < n; ++i) p[i] = fill ? unif() : 0.0;
  return p;
}
static void finite(const char *what, const double *p, long n) {
  for (long i = 0; i < n; ++i)
    if (!isfinite(p[i])) {
      printf("non-finite %s[%ld]\n", what, i);
      ++failures;
      return;
    }
}

static void run(long B, long H, long N, long D, long M, long fm) {
  const long BH = B * H, nq = BH * N * D, nv = BH * N * M, ns = BH * D * M, nz = BH * D;
  double *Q = arr(nq, 1), *K = arr(nq, 1), *V = arr(nv, 1), *dO = arr(nv, 1), *logA = arr(BH * N, 1);
  double *S0 = arr(ns, 1), *Z0 = arr(nz, 0), *dSN = arr(ns, 1), *dZN = arr(nz, 1);
  for (long i = 0; i < BH * N; ++i) logA[i] = -0.5 * (logA[i] + 1.0); /* in (-1, 0] */
  for (long i = 0; i < nz; ++i) Z0[i] = 1.0 + 0.5 * unif();         /* a state of positive features */
  if (fm) /* feature mode: Q, K are feature vectors, kept positive */
    for (long i = 0; i < nq; ++i) {
      Q[i] = 1.5 + Q[i];
      K[i] = 1.5 + K[i];
    }
  double *O = arr(nv, 0), *den = arr(BH * N, 0), *S = arr(ns, 0), *Z = arr(nz, 0);
  double *dQ = arr(nq, 0), *dK = arr(nq, 0), *dV = arr(nv, 0), *dS0 = arr(ns, 0), *dZ0 = arr(nz, 0);
  double *dla = arr(BH * N, 0), *P = arr(BH * N * N, 0);

  orc_forward_causal(Q, K, V, NULL, NULL, O, NULL, NULL, NULL, B, H, N, D, M, fm);
  orc_forward_causal(Q, K, V, S0, Z0, O, den, S, Z, B, H, N, D, M, fm);
  finite("O", O, nv);
  finite("S", S, ns);
  if (!fm) { /* the quadratic form always applies eq. 7 */
    orc_forward_causal_parallel(Q, K, V, O, den, B, H, N, D, M);
    finite("O parallel", O, nv);
  }
  orc_forward_noncausal(Q, K, V, O, B, H, N, D, M, fm);
  finite("O non-causal", O, nv);
  orc_backward_causal(Q, K, V, dO, NULL, NULL, NULL, NULL, dQ, dK, dV, NULL, NULL, B, H, N, D, M, fm);
  orc_backward_causal(Q, K, V, dO, S0, Z0, dSN, dZN, dQ, dK, dV, dS0, dZ0, B, H, N, D, M, fm);
  finite("dQ", dQ, nq);
  finite("dS0", dS0, ns);
  orc_backward_noncausal(Q, K, V, dO, dQ, dK, dV, B, H, N, D, M, fm);
  finite("dK non-causal", dK, nq);
  orc_forward_decay(Q, K, V, logA, NULL, NULL, O, NULL, NULL, NULL, B, H, N, D, M, fm);
  orc_forward_decay(Q, K, V, logA, S0, Z0, O, den, S, Z, B, H, N, D, M, fm);
  finite("O decay", O, nv);
  orc_backward_decay(Q, K, V, logA, dO, NULL, NULL, NULL, NULL, dQ, dK, dV, dla, NULL, NULL, B, H, N, D, M, fm);
  orc_backward_decay(Q, K, V, logA, dO, S0, Z0, dSN, dZN, dQ, dK, dV, dla, dS0, dZ0, B, H, N, D, M, fm);
  finite("dlogA", dla, BH * N);
  if (N > 0) { /* decode on the first token of every head, from (S0, Z0), without and with a decay */
    double *q = arr(nz, 0), *k = arr(nz, 0), *v = arr(BH * M, 0), *y = arr(BH * M, 0), *a = arr(BH, 0);
    for (long bh = 0; bh < BH; ++bh) {
      for (long d = 0; d < D; ++d) {
        q[bh * D + d] = Q[bh * N * D + d];
        k[bh * D + d] = K[bh * N * D + d];
      }
      for (long m = 0; m < M; ++m) v[bh * M + m] = V[bh * N * M + m];
      a[bh] = logA[bh * N];
    }
    for (long i = 0; i < ns; ++i) S[i] = S0[i];
    for (long i = 0; i < nz; ++i) Z[i] = Z0[i];
    orc_decode_step(q, k, v, NULL, S, Z, y, B, H, D, M, fm);
    orc_decode_step(q, k, v, a, S, Z, y, B, H, D, M, fm);
    finite("y", y, BH * M);
    free(q); free(k); free(v); free(y); free(a);
  }
  /* constant rows of V: every output row is that row */
  for (long bh = 0; bh < BH; ++bh)
    for (long i = 0; i < N; ++i)
      for (long m = 0; m < M; ++m) V[(bh * N + i) * M + m] = V[bh * N * M + m];
  for (int causal = 0; causal < 2; ++causal) {
    if (causal)
      orc_forward_causal(Q, K, V, NULL, NULL, O, NULL, NULL, NULL, B, H, N, D, M, fm);
    else
      orc_forward_noncausal(Q, K, V, O, B, H, N, D, M, fm);
    for (long e = 0; e < nv; ++e) {
      const long bh = e / (N * M), m = e % M;
      if (fabs(O[e] - V[bh * N * M + m]) > 1e-12 * (1.0 + fabs(V[bh * N * M + m]))) {
        printf("constant-V rows: O[%ld] = %.17g, expected %.17g (causal %d)\n", e, O[e], V[bh * N * M + m], causal);
        ++failures;
        break;
      }
    }
  }
  free(Q); free(K); free(V); free(dO); free(logA); free(S0); free(Z0); free(dSN); free(dZN);
  free(O); free(den); free(S); free(Z); free(dQ); free(dK); free(dV); free(dS0); free(dZ0); free(dla); free(P);
}

static void run_features(long B, long H, long N, long Din, long C) {
  const long rows = B * H * N;
  double *X = arr(rows * Din, 1), *W = arr(H * C * Din, 1), *Phi = arr(rows * C, 0), *dPhi = arr(rows * C, 1);
  double *dX = arr(rows * Din, 0);
  orc_feature_performer(X, W, Phi, B, H, N, Din, C);
  finite("Phi", Phi, rows * C);
  orc_feature_performer_vjp(X, W, dPhi, dX, B, H, N, Din, C);
  finite("dX", dX, rows * Din);
  const long Cp = 1 + Din + Din * Din;
  double *Pp = arr(rows * Cp, 0), *dPp = arr(rows * Cp, 1);
  orc_feature_poly2(X, Pp, rows, Din, Cp);
  orc_feature_poly2_vjp(X, dPp, dX, rows, Din, Cp);
  finite("dX poly2", dX, rows * Din);
  free(X); free(W); free(Phi); free(dPhi); free(dX); free(Pp); free(dPp);
}

int main(void) {
  static const long shapes[][5] = {{1, 1, 0, 3, 4}, {1, 1, 1, 3, 4}, {2, 3, 17, 5, 4}, {1, 2, 9, 4, 7}, {2, 1, 33, 8, 8}};
  for (unsigned s = 0; s < sizeof(shapes) / sizeof(shapes[0]); ++s)
    for (long fm = 0; fm < 2; ++fm) run(shapes[s][0], shapes[s][1], shapes[s][2], shapes[s][3], shapes[s][4], fm);
  run_features(1, 1, 1, 3, 5);
  run_features(2, 3, 11, 4, 6);
  printf("%s (%d failures)\n", failures ? "FAILED" : "ok", failures);
  return failures ? 1 : 0;
}
