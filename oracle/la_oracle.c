/*
 * la_oracle.c -- float64 CPU oracle for causal linear attention with
 * phi(x) = elu(x) + 1.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path links, loads or
 * calls this file: only the test-suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or table with the HIP
 * library.
 *
 * Every routine is the plain definition written out, in float64, one token
 * at a time; there is no chunking, blocking or fusion.  The attention
 * routines take a last argument fm: 0 applies eq. 7 to Q and K, 1 takes them
 * as feature vectors already (the feature maps at the end of this file).  Parallelism is only
 * across independent (batch, head) pairs (heads never interact: Transformer
 * Family v2, multi-head attention section).
 *
 * Sources, cited by page title and equation:
 *  [TaR]  "Transformers are RNNs: Fast Autoregressive Transformers with
 *         Linear Attention -- part 2/3": eq. 7 (feature map), eq. 8-12
 *         (causal masking), eq. 13-15 (gradient of the numerator), eq. 16-20
 *         (the RNN form).
 *  [TaRn] reading notes "Transformers are RNNs" (papercache): section 3.2
 *         eq. 4-6 (non-causal linearised attention), appendix A (the
 *         denominator's gradient left to automatic differentiation).
 *  [LA]   "Linear Attention/zh": kernel reformulation (S, z summed once and
 *         reused), recurrent form (S_t, z_t updates).
 *
 * Readings where the pages leave a step open:
 *  - elu's alpha is 1 (the Clevert et al. default the pages cite), so
 *    phi(x) = x + 1 for x > 0 and exp(x) otherwise; phi'(x) = 1 for x > 0
 *    and exp(x) otherwise.
 *  - no epsilon in the denominator.
 *  - causal masking is inclusive (j <= i), as eq. 8 states.
 *  - the gradient of the denominator and of the fraction, left by the pages
 *    to autograd, is the quotient rule: with num_i and den_i the numerator
 *    and denominator of eq. 12 and dO_i the upstream gradient,
 *      d num_i = dO_i / den_i,   d den_i = -(dO_i . O_i) / den_i.
 *    The denominator of eq. 12 is the numerator with V replaced by a column
 *    of ones, so both are handled by the numerator gradient of eq. 13-15
 *    applied to V-bar = [V, 1] with upstream [d num, d den].
 *  - gradients are returned with respect to the raw Q, K, V (chain rule
 *    through phi').
 *
 * All pins of these routines are structural (the pages print no tensor
 * values); they live in the test-suite.
 *
 * Layout: row-major, Q and K [B,H,N,D]; V, O, dO [B,H,N,M]; den [B,H,N];
 * S [B,H,D,M] with S[d][m] = sum_j phi(K_j)[d] V_j[m]; Z [B,H,D].
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>

/* [TaR] eq. 7 with alpha = 1. */
double orc_phi(double x) { return x > 0.0 ? x + 1.0 : exp(x); }

/* Derivative of eq. 7: 1 for x > 0, exp(x) otherwise (both sides give 1 at 0). */
double orc_dphi(double x) { return x > 0.0 ? 1.0 : exp(x); }

/* Feature-map selection of every attention routine: fm = 0 applies eq. 7 to
 * Q and K; fm = 1 takes them as feature vectors already (another feature map
 * applied beforehand, "Linear Attention/zh", feature maps), i.e. the identity
 * with derivative 1, and the gradients are with respect to those features. */
static double feat(double x, long fm) { return fm ? x : orc_phi(x); }
static double dfeat(double x, long fm) { return fm ? 1.0 : orc_dphi(x); }

/*
 * Causal forward, recurrent form ([TaR] eq. 10-12, eq. 16-19 without the
 * projections):  S_i = S_{i-1} + phi(K_i) V_i^T,  Z_i = Z_{i-1} + phi(K_i),
 * den_i = phi(Q_i) . Z_i,  O_i = phi(Q_i)^T S_i / den_i.
 * S0/Z0 (both or neither, may be NULL) are the state before token 1.
 * den, S_out, Z_out may be NULL.
 */
void orc_forward_causal(const double *Q, const double *K, const double *V,
                        const double *S0, const double *Z0, double *O,
                        double *den, double *S_out, double *Z_out, long B,
                        long H, long N, long D, long M, long fm) {
  long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    double *S = (double *)calloc((size_t)(D * M), sizeof(double));
    double *Z = (double *)calloc((size_t)D, sizeof(double));
    double *pq = (double *)malloc((size_t)D * sizeof(double));
    double *pk = (double *)malloc((size_t)D * sizeof(double));
    if (S0) memcpy(S, S0 + bh * D * M, (size_t)(D * M) * sizeof(double));
    if (Z0) memcpy(Z, Z0 + bh * D, (size_t)D * sizeof(double));
    for (long i = 0; i < N; ++i) {
      const double *q = Q + (bh * N + i) * D;
      const double *k = K + (bh * N + i) * D;
      const double *v = V + (bh * N + i) * M;
      for (long d = 0; d < D; ++d) {
        pq[d] = feat(q[d], fm);
        pk[d] = feat(k[d], fm);
      }
      /* state update first: the mask is inclusive (eq. 8, j <= i) */
      for (long d = 0; d < D; ++d) {
        for (long m = 0; m < M; ++m) S[d * M + m] += pk[d] * v[m];
        Z[d] += pk[d];
      }
      double dn = 0.0;
      for (long d = 0; d < D; ++d) dn += pq[d] * Z[d];
      double *o = O + (bh * N + i) * M;
      for (long m = 0; m < M; ++m) {
        double num = 0.0;
        for (long d = 0; d < D; ++d) num += pq[d] * S[d * M + m];
        o[m] = num / dn;
      }
      if (den) den[bh * N + i] = dn;
    }
    if (S_out) memcpy(S_out + bh * D * M, S, (size_t)(D * M) * sizeof(double));
    if (Z_out) memcpy(Z_out + bh * D, Z, (size_t)D * sizeof(double));
    free(S);
    free(Z);
    free(pq);
    free(pk);
  }
}

/*
 * Causal forward, parallel (quadratic) form ([TaR] eq. 9 read as matrices):
 * A = phi(Q) phi(K)^T with the inclusive lower-triangular mask,
 * O = (A V) / (A 1) row-wise.  Cross-check for the recurrent form; O(N^2).
 */
void orc_forward_causal_parallel(const double *Q, const double *K,
                                 const double *V, double *O, double *den,
                                 long B, long H, long N, long D, long M) {
  long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    double *pq = (double *)malloc((size_t)(N * D) * sizeof(double));
    double *pk = (double *)malloc((size_t)(N * D) * sizeof(double));
    double *arow = (double *)malloc((size_t)N * sizeof(double));
    for (long t = 0; t < N * D; ++t) {
      pq[t] = orc_phi(Q[bh * N * D + t]);
      pk[t] = orc_phi(K[bh * N * D + t]);
    }
    for (long i = 0; i < N; ++i) {
      double rowsum = 0.0;
      for (long j = 0; j <= i; ++j) {
        double a = 0.0;
        for (long d = 0; d < D; ++d) a += pq[i * D + d] * pk[j * D + d];
        arow[j] = a;
        rowsum += a;
      }
      double *o = O + (bh * N + i) * M;
      for (long m = 0; m < M; ++m) {
        double acc = 0.0;
        for (long j = 0; j <= i; ++j) acc += arow[j] * V[(bh * N + j) * M + m];
        o[m] = acc / rowsum;
      }
      if (den) den[bh * N + i] = rowsum;
    }
    free(pq);
    free(pk);
    free(arow);
  }
}

/*
 * Non-causal forward ([TaRn] section 3.2, eq. 5-6; [LA] kernel
 * reformulation): S = sum_j phi(K_j) V_j^T and Z = sum_j phi(K_j) are formed
 * once per head and reused for every query: O_i = phi(Q_i)^T S / phi(Q_i).Z.
 */
void orc_forward_noncausal(const double *Q, const double *K, const double *V,
                           double *O, long B, long H, long N, long D, long M, long fm) {
  long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    double *S = (double *)calloc((size_t)(D * M), sizeof(double));
    double *Z = (double *)calloc((size_t)D, sizeof(double));
    double *pq = (double *)malloc((size_t)D * sizeof(double));
    for (long j = 0; j < N; ++j) {
      const double *k = K + (bh * N + j) * D;
      const double *v = V + (bh * N + j) * M;
      for (long d = 0; d < D; ++d) {
        double pk = feat(k[d], fm);
        for (long m = 0; m < M; ++m) S[d * M + m] += pk * v[m];
        Z[d] += pk;
      }
    }
    for (long i = 0; i < N; ++i) {
      const double *q = Q + (bh * N + i) * D;
      for (long d = 0; d < D; ++d) pq[d] = feat(q[d], fm);
      double dn = 0.0;
      for (long d = 0; d < D; ++d) dn += pq[d] * Z[d];
      double *o = O + (bh * N + i) * M;
      for (long m = 0; m < M; ++m) {
        double num = 0.0;
        for (long d = 0; d < D; ++d) num += pq[d] * S[d * M + m];
        o[m] = num / dn;
      }
    }
    free(S);
    free(Z);
    free(pq);
  }
}

/*
 * Gradient of the causal numerator ([TaR] eq. 13-15) for one head.
 * Inputs are already feature-mapped, as the pages' appendix allows
 * ("without loss of generality Q and K already hold phi-mapped vectors"):
 *   P = phi(Q) [N,C], Kf = phi(K) [N,C], Vb [N,Mb], G = dL/dVbar [N,Mb]
 * where Vbar_i = sum_{j<=i} (P_i . Kf_j) Vb_j.
 *   eq. 13: dP_i  = S_i G_i,      S_i = sum_{j<=i} Kf_j Vb_j^T   (forward sum)
 *   eq. 14: dKf_i = R_i Vb_i,     R_i = sum_{j>=i} P_j G_j^T     (reverse sum)
 *   eq. 15: dVb_i = R_i^T Kf_i.
 * The two sums are accumulated token by token in opposite directions.
 *
 * State gradients.  The state after the last token, S_N = S_0 +
 * sum_j Kf_j Vb_j^T, may itself feed the loss with upstream gradient RN
 * [C,Mb] (NULL: zero).  Every term Kf_j Vb_j^T is part of S_N, so RN is the
 * starting value of the reverse sum: R_i = RN + sum_{j>=i} P_j G_j^T.  The
 * initial state S_0 is part of every S_i and of S_N, so its gradient is the
 * reverse sum carried through token 1, R0 = RN + sum_j P_j G_j^T (output when
 * R0 is not NULL; equal to RN for N = 0).
 */
void orc_numerator_backward(const double *P, const double *Kf, const double *Vb,
                            const double *G, const double *RN, double *dP,
                            double *dKf, double *dVb, double *R0, long N,
                            long C, long Mb) {
  double *S = (double *)calloc((size_t)(C * Mb), sizeof(double));
  double *R = (double *)calloc((size_t)(C * Mb), sizeof(double));
  if (RN) memcpy(R, RN, (size_t)(C * Mb) * sizeof(double));
  for (long i = 0; i < N; ++i) { /* forward cumulative sum, eq. 13 */
    for (long c = 0; c < C; ++c)
      for (long m = 0; m < Mb; ++m) S[c * Mb + m] += Kf[i * C + c] * Vb[i * Mb + m];
    for (long c = 0; c < C; ++c) {
      double acc = 0.0;
      for (long m = 0; m < Mb; ++m) acc += S[c * Mb + m] * G[i * Mb + m];
      dP[i * C + c] = acc;
    }
  }
  for (long i = N - 1; i >= 0; --i) { /* reverse cumulative sum, eq. 14-15 */
    for (long c = 0; c < C; ++c)
      for (long m = 0; m < Mb; ++m) R[c * Mb + m] += P[i * C + c] * G[i * Mb + m];
    for (long c = 0; c < C; ++c) {
      double acc = 0.0;
      for (long m = 0; m < Mb; ++m) acc += R[c * Mb + m] * Vb[i * Mb + m];
      dKf[i * C + c] = acc;
    }
    for (long m = 0; m < Mb; ++m) {
      double acc = 0.0;
      for (long c = 0; c < C; ++c) acc += R[c * Mb + m] * Kf[i * C + c];
      dVb[i * Mb + m] = acc;
    }
  }
  if (R0) memcpy(R0, R, (size_t)(C * Mb) * sizeof(double));
  free(S);
  free(R);
}

/*
 * Full causal backward: gradients of L = sum(dO * O) with respect to the raw
 * Q, K, V, where O is the causal forward of eq. 12 started from (S0, Z0)
 * (both may be NULL: zero state).  The loss may also depend on the final
 * state (S_N, Z_N) of eq. 10-11 with upstream gradients dSN [B,H,D,M],
 * dZN [B,H,D] (both or neither, NULL: zero); then dS0 [B,H,D,M] and
 * dZ0 [B,H,D] (both or neither, may be NULL) receive the gradient with
 * respect to the initial state.  Steps:
 *  1. forward recurrence (eq. 10-12) for den_i and O_i;
 *  2. quotient rule: d num_i = dO_i / den_i, d den_i = -(dO_i . O_i) / den_i;
 *  3. eq. 13-15 on the augmented values Vbar = [V, 1] with upstream
 *     [d num, d den] (the denominator is the numerator of a ones column, and
 *     Z is the state of that column, so [S | Z] is the augmented state and
 *     [dSN | dZN] its final gradient); an initial state contributes S0 G_i to
 *     the phi(Q) gradient (it is the j = 0 term of the forward sum of
 *     eq. 13), and receives the reverse sum carried through token 1;
 *  4. chain rule through phi: dQ = dphiQ * phi'(Q), dK = dphiK * phi'(K).
 */
void orc_backward_causal(const double *Q, const double *K, const double *V,
                         const double *dO, const double *S0, const double *Z0,
                         const double *dSN, const double *dZN, double *dQ,
                         double *dK, double *dV, double *dS0, double *dZ0,
                         long B, long H, long N, long D, long M, long fm) {
  long BH = B * H;
  long Mb = M + 1;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    const double *q = Q + bh * N * D, *k = K + bh * N * D, *v = V + bh * N * M;
    const double *go = dO + bh * N * M;
    double *O = (double *)malloc((size_t)(N * M) * sizeof(double));
    double *den = (double *)malloc((size_t)N * sizeof(double));
    double *P = (double *)malloc((size_t)(N * D) * sizeof(double));
    double *Kf = (double *)malloc((size_t)(N * D) * sizeof(double));
    double *Vb = (double *)malloc((size_t)(N * Mb) * sizeof(double));
    double *G = (double *)malloc((size_t)(N * Mb) * sizeof(double));
    double *dP = (double *)malloc((size_t)(N * D) * sizeof(double));
    double *dKf = (double *)malloc((size_t)(N * D) * sizeof(double));
    double *dVb = (double *)malloc((size_t)(N * Mb) * sizeof(double));
    double *RN = (double *)calloc((size_t)(D * Mb), sizeof(double));
    double *R0 = (double *)malloc((size_t)(D * Mb) * sizeof(double));
    if (dSN)
      for (long d = 0; d < D; ++d) {
        for (long m = 0; m < M; ++m) RN[d * Mb + m] = dSN[bh * D * M + d * M + m];
        RN[d * Mb + M] = dZN[bh * D + d];
      }
    /* 1. forward pass of this head */
    orc_forward_causal(q, k, v, S0 ? S0 + bh * D * M : NULL,
                       Z0 ? Z0 + bh * D : NULL, O, den, NULL, NULL, 1, 1, N, D, M, fm);
    /* 2. quotient rule, 3. augmented numerator */
    for (long i = 0; i < N; ++i) {
      for (long d = 0; d < D; ++d) {
        P[i * D + d] = feat(q[i * D + d], fm);
        Kf[i * D + d] = feat(k[i * D + d], fm);
      }
      double dot = 0.0;
      for (long m = 0; m < M; ++m) {
        Vb[i * Mb + m] = v[i * M + m];
        G[i * Mb + m] = go[i * M + m] / den[i];
        dot += go[i * M + m] * O[i * M + m];
      }
      Vb[i * Mb + M] = 1.0;
      G[i * Mb + M] = -dot / den[i];
    }
    orc_numerator_backward(P, Kf, Vb, G, RN, dP, dKf, dVb, R0, N, D, Mb);
    if (dS0)
      for (long d = 0; d < D; ++d) {
        for (long m = 0; m < M; ++m) dS0[bh * D * M + d * M + m] = R0[d * Mb + m];
        dZ0[bh * D + d] = R0[d * Mb + M];
      }
    if (S0 || Z0) { /* initial state: the j = 0 term of eq. 13's sum */
      for (long i = 0; i < N; ++i)
        for (long d = 0; d < D; ++d) {
          double acc = 0.0;
          for (long m = 0; m < M; ++m)
            acc += (S0 ? S0[bh * D * M + d * M + m] : 0.0) * G[i * Mb + m];
          acc += (Z0 ? Z0[bh * D + d] : 0.0) * G[i * Mb + M];
          dP[i * D + d] += acc;
        }
    }
    /* 4. chain rule through phi */
    for (long i = 0; i < N; ++i) {
      for (long d = 0; d < D; ++d) {
        dQ[(bh * N + i) * D + d] = dP[i * D + d] * dfeat(q[i * D + d], fm);
        dK[(bh * N + i) * D + d] = dKf[i * D + d] * dfeat(k[i * D + d], fm);
      }
      for (long m = 0; m < M; ++m) dV[(bh * N + i) * M + m] = dVb[i * Mb + m];
    }
    free(O);
    free(den);
    free(P);
    free(Kf);
    free(Vb);
    free(G);
    free(dP);
    free(dKf);
    free(dVb);
    free(RN);
    free(R0);
  }
}

/*
 * Non-causal backward: gradients of L = sum(dO * O) with respect to the raw
 * Q, K, V for the non-causal forward ([TaRn] section 3.2, eq. 5-6), where
 * every query sees every key.  The same steps as the causal backward with
 * the masks removed, so the cumulative sums of eq. 13-15 become totals:
 *  1. S = sum_j phi(K_j) V_j^T, Z = sum_j phi(K_j); den_i = phi(Q_i) . Z,
 *     O_i = phi(Q_i)^T S / den_i;
 *  2. quotient rule: g_i = dO_i / den_i, c_i = -(dO_i . O_i) / den_i;
 *  3. on [V, 1] with upstream [g, c]:
 *       dphiQ_i = S g_i + c_i Z                    (eq. 13 with S_i = S),
 *       R = sum_i phi(Q_i) g_i^T, r = sum_i c_i phi(Q_i)   (eq. 14's sum over all i),
 *       dphiK_j = R V_j + r,  dV_j = R^T phi(K_j)  (eq. 14-15);
 *  4. chain rule through phi.
 */
void orc_backward_noncausal(const double *Q, const double *K, const double *V,
                            const double *dO, double *dQ, double *dK,
                            double *dV, long B, long H, long N, long D,
                            long M, long fm) {
  long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    const double *q = Q + bh * N * D, *k = K + bh * N * D, *v = V + bh * N * M;
    const double *go = dO + bh * N * M;
    double *S = (double *)calloc((size_t)(D * M), sizeof(double));
    double *Z = (double *)calloc((size_t)D, sizeof(double));
    double *R = (double *)calloc((size_t)(D * M), sizeof(double));
    double *r = (double *)calloc((size_t)D, sizeof(double));
    double *pq = (double *)malloc((size_t)D * sizeof(double));
    double *g = (double *)malloc((size_t)M * sizeof(double));
    /* 1. totals of the keys */
    for (long j = 0; j < N; ++j)
      for (long d = 0; d < D; ++d) {
        double pk = feat(k[j * D + d], fm);
        for (long m = 0; m < M; ++m) S[d * M + m] += pk * v[j * M + m];
        Z[d] += pk;
      }
    /* 2-3. per query: den, O, g, c; dphiQ; accumulate R, r */
    for (long i = 0; i < N; ++i) {
      for (long d = 0; d < D; ++d) pq[d] = feat(q[i * D + d], fm);
      double den = 0.0;
      for (long d = 0; d < D; ++d) den += pq[d] * Z[d];
      double dot = 0.0;
      for (long m = 0; m < M; ++m) {
        double num = 0.0;
        for (long d = 0; d < D; ++d) num += pq[d] * S[d * M + m];
        dot += go[i * M + m] * (num / den);
        g[m] = go[i * M + m] / den;
      }
      double c = -dot / den;
      for (long d = 0; d < D; ++d) {
        double acc = c * Z[d];
        for (long m = 0; m < M; ++m) acc += S[d * M + m] * g[m];
        dQ[(bh * N + i) * D + d] = acc * dfeat(q[i * D + d], fm);
        for (long m = 0; m < M; ++m) R[d * M + m] += pq[d] * g[m];
        r[d] += c * pq[d];
      }
    }
    /* 3-4. per key */
    for (long j = 0; j < N; ++j) {
      for (long d = 0; d < D; ++d) {
        double acc = r[d];
        for (long m = 0; m < M; ++m) acc += R[d * M + m] * v[j * M + m];
        dK[(bh * N + j) * D + d] = acc * dfeat(k[j * D + d], fm);
      }
      for (long m = 0; m < M; ++m) {
        double acc = 0.0;
        for (long d = 0; d < D; ++d) acc += R[d * M + m] * feat(k[j * D + d], fm);
        dV[(bh * N + j) * M + m] = acc;
      }
    }
    free(S);
    free(Z);
    free(R);
    free(r);
    free(pq);
    free(g);
  }
}

/*
 * Decayed causal forward ([LA] "Variants and extensions": RetNet replaces
 * the unbounded cumulative sum by S_t = gamma S_{t-1} + phi(k_t) v_t^T with
 * gamma in (0, 1); gated linear attention makes the decay data-dependent).
 * Here the decay is one scalar per token and head, given by its logarithm
 * logA [B,H,N] (a_t = exp(logA_t) in (0, 1]; a constant per head is the
 * RetNet case).  The pages give the update of S only; the normaliser Z takes
 * the same decay, so that the output stays a weighted average of the values:
 *   S_t = a_t S_{t-1} + phi(K_t) V_t^T,  Z_t = a_t Z_{t-1} + phi(K_t),
 *   den_t = phi(Q_t) . Z_t,  O_t = phi(Q_t)^T S_t / den_t.
 * With logA = 0 this is orc_forward_causal.  S0/Z0 (both or neither) are the
 * state before token 1 (decayed by a_1 like any earlier state); den, S_out,
 * Z_out may be NULL.
 */
void orc_forward_decay(const double *Q, const double *K, const double *V,
                       const double *logA, const double *S0, const double *Z0,
                       double *O, double *den, double *S_out, double *Z_out,
                       long B, long H, long N, long D, long M, long fm) {
  long BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    double *S = (double *)calloc((size_t)(D * M), sizeof(double));
    double *Z = (double *)calloc((size_t)D, sizeof(double));
    double *pq = (double *)malloc((size_t)D * sizeof(double));
    double *pk = (double *)malloc((size_t)D * sizeof(double));
    if (S0) memcpy(S, S0 + bh * D * M, (size_t)(D * M) * sizeof(double));
    if (Z0) memcpy(Z, Z0 + bh * D, (size_t)D * sizeof(double));
    for (long i = 0; i < N; ++i) {
      const double *q = Q + (bh * N + i) * D;
      const double *k = K + (bh * N + i) * D;
      const double *v = V + (bh * N + i) * M;
      const double a = exp(logA[bh * N + i]);
      for (long d = 0; d < D; ++d) {
        pq[d] = feat(q[d], fm);
        pk[d] = feat(k[d], fm);
      }
      for (long d = 0; d < D; ++d) {
        for (long m = 0; m < M; ++m) S[d * M + m] = a * S[d * M + m] + pk[d] * v[m];
        Z[d] = a * Z[d] + pk[d];
      }
      double dn = 0.0;
      for (long d = 0; d < D; ++d) dn += pq[d] * Z[d];
      double *o = O + (bh * N + i) * M;
      for (long m = 0; m < M; ++m) {
        double num = 0.0;
        for (long d = 0; d < D; ++d) num += pq[d] * S[d * M + m];
        o[m] = num / dn;
      }
      if (den) den[bh * N + i] = dn;
    }
    if (S_out) memcpy(S_out + bh * D * M, S, (size_t)(D * M) * sizeof(double));
    if (Z_out) memcpy(Z_out + bh * D, Z, (size_t)D * sizeof(double));
    free(S);
    free(Z);
    free(pq);
    free(pk);
  }
}

/*
 * Backward of orc_forward_decay: reverse-mode differentiation of its
 * recurrence, token by token.  The loss is sum(dO * O) + sum(dSN * S_N) +
 * sum(dZN * Z_N) (dSN/dZN both or neither, NULL: zero).  With the augmented
 * state Sb_t = [S_t | Z_t] (D x (M+1)), the augmented value [V_t, 1] and the
 * quotient rule's upstream Gb_t = [dO_t / den_t, -(dO_t . O_t) / den_t]:
 *   R = [dSN | dZN];  for t = N .. 1:
 *     R += phi(Q_t) Gb_t^T               (the gradient of Sb_t is complete)
 *     dphiQ_t = Sb_t Gb_t,  dphiK_t = R [V_t, 1],  dV_t = (R^T phi(K_t))[:M]
 *     dlogA_t = a_t <R, Sb_{t-1}>        (Sb_t depends on a_t through a_t Sb_{t-1})
 *     R = a_t R                          (the gradient of Sb_{t-1})
 *   [dS0 | dZ0] = R.
 * then the chain rule through phi.  The forward states Sb_0 .. Sb_N are kept
 * (O(N D M) memory per head: this is the oracle, not the product).
 * dS0/dZ0 (both or neither) may be NULL.
 */
void orc_backward_decay(const double *Q, const double *K, const double *V,
                        const double *logA, const double *dO,
                        const double *S0, const double *Z0, const double *dSN,
                        const double *dZN, double *dQ, double *dK, double *dV,
                        double *dlogA, double *dS0, double *dZ0, long B, long H,
                        long N, long D, long M, long fm) {
  long BH = B * H;
  long Mb = M + 1, SB = D * (M + 1);
#pragma omp parallel for schedule(dynamic, 1)
  for (long bh = 0; bh < BH; ++bh) {
    const double *q = Q + bh * N * D, *k = K + bh * N * D, *v = V + bh * N * M;
    const double *go = dO + bh * N * M, *la = logA + bh * N;
    double *Sb = (double *)calloc((size_t)((N + 1) * SB), sizeof(double));
    double *R = (double *)calloc((size_t)SB, sizeof(double));
    double *pq = (double *)malloc((size_t)D * sizeof(double));
    double *pk = (double *)malloc((size_t)D * sizeof(double));
    double *G = (double *)malloc((size_t)Mb * sizeof(double));
    /* forward: Sb_0 = [S0 | Z0], Sb_t = a_t Sb_{t-1} + phi(K_t) [V_t, 1]^T */
    for (long d = 0; d < D; ++d) {
      for (long m = 0; m < M; ++m) Sb[d * Mb + m] = S0 ? S0[bh * D * M + d * M + m] : 0.0;
      Sb[d * Mb + M] = Z0 ? Z0[bh * D + d] : 0.0;
    }
    for (long t = 1; t <= N; ++t) {
      const double a = exp(la[t - 1]);
      const double *prev = Sb + (t - 1) * SB;
      double *cur = Sb + t * SB;
      for (long d = 0; d < D; ++d) {
        const double p = feat(k[(t - 1) * D + d], fm);
        for (long m = 0; m < M; ++m) cur[d * Mb + m] = a * prev[d * Mb + m] + p * v[(t - 1) * M + m];
        cur[d * Mb + M] = a * prev[d * Mb + M] + p;
      }
    }
    if (dSN)
      for (long d = 0; d < D; ++d) {
        for (long m = 0; m < M; ++m) R[d * Mb + m] = dSN[bh * D * M + d * M + m];
        R[d * Mb + M] = dZN[bh * D + d];
      }
    for (long t = N; t >= 1; --t) {
      const long i = t - 1;
      const double a = exp(la[i]);
      const double *cur = Sb + t * SB, *prev = Sb + (t - 1) * SB;
      for (long d = 0; d < D; ++d) {
        pq[d] = feat(q[i * D + d], fm);
        pk[d] = feat(k[i * D + d], fm);
      }
      /* output of token t and the quotient rule */
      double dn = 0.0;
      for (long d = 0; d < D; ++d) dn += pq[d] * cur[d * Mb + M];
      double dot = 0.0;
      for (long m = 0; m < M; ++m) {
        double num = 0.0;
        for (long d = 0; d < D; ++d) num += pq[d] * cur[d * Mb + m];
        dot += go[i * M + m] * (num / dn);
        G[m] = go[i * M + m] / dn;
      }
      G[M] = -dot / dn;
      for (long d = 0; d < D; ++d)
        for (long m = 0; m < Mb; ++m) R[d * Mb + m] += pq[d] * G[m];
      for (long d = 0; d < D; ++d) {
        double aq = 0.0, ak = R[d * Mb + M];
        for (long m = 0; m < Mb; ++m) aq += cur[d * Mb + m] * G[m];
        for (long m = 0; m < M; ++m) ak += R[d * Mb + m] * v[i * M + m];
        dQ[(bh * N + i) * D + d] = aq * dfeat(q[i * D + d], fm);
        dK[(bh * N + i) * D + d] = ak * dfeat(k[i * D + d], fm);
      }
      for (long m = 0; m < M; ++m) {
        double acc = 0.0;
        for (long d = 0; d < D; ++d) acc += R[d * Mb + m] * pk[d];
        dV[(bh * N + i) * M + m] = acc;
      }
      double ip = 0.0;
      for (long e = 0; e < SB; ++e) ip += R[e] * prev[e];
      dlogA[bh * N + i] = a * ip;
      for (long e = 0; e < SB; ++e) R[e] *= a;
    }
    if (dS0)
      for (long d = 0; d < D; ++d) {
        for (long m = 0; m < M; ++m) dS0[bh * D * M + d * M + m] = R[d * Mb + m];
        dZ0[bh * D + d] = R[d * Mb + M];
      }
    free(Sb);
    free(R);
    free(pq);
    free(pk);
    free(G);
  }
}

/*
 * One RNN decode step ([TaR] eq. 18-20, attention part; [LA] recurrent
 * form): S = a S + phi(k) v^T, Z = a Z + phi(k), then y = phi(q)^T S /
 * phi(q).Z, with a = exp(logA) per (batch, head) for the decayed recurrence
 * of orc_forward_decay, and a = 1 when logA is NULL.
 * S [B,H,D,M] and Z [B,H,D] are updated in place; y [B,H,M].
 */
void orc_decode_step(const double *q, const double *k, const double *v,
                     const double *logA, double *S, double *Z, double *y,
                     long B, long H, long D, long M, long fm) {
  long BH = B * H;
#pragma omp parallel for schedule(static)
  for (long bh = 0; bh < BH; ++bh) {
    double *s = S + bh * D * M, *z = Z + bh * D;
    const double a = logA ? exp(logA[bh]) : 1.0;
    for (long d = 0; d < D; ++d) {
      double pk = feat(k[bh * D + d], fm);
      for (long m = 0; m < M; ++m) s[d * M + m] = a * s[d * M + m] + pk * v[bh * M + m];
      z[d] = a * z[d] + pk;
    }
    double dn = 0.0;
    for (long d = 0; d < D; ++d) dn += feat(q[bh * D + d], fm) * z[d];
    for (long m = 0; m < M; ++m) {
      double num = 0.0;
      for (long d = 0; d < D; ++d) num += feat(q[bh * D + d], fm) * s[d * M + m];
      y[bh * M + m] = num / dn;
    }
  }
}

/*
 * Positive random features ("Linear Attention/zh", feature maps: Performer
 * approximates the softmax kernel with phi(x) proportional to
 * exp(W x - |x|^2 / 2); "The Transformer Family v2", random feature
 * attention).  With a projection W [C, Din] per head (random, passed in):
 *   phi(x)_c = exp(w_c . x - |x|^2 / 2) / sqrt(C),
 * so phi(x) . phi(y) = mean_c exp(w_c . (x + y) - (|x|^2 + |y|^2) / 2),
 * whose expectation over standard normal w_c is exp(x . y).
 * X [B,H,N,Din], W [H,C,Din], Phi [B,H,N,C].
 */
void orc_feature_performer(const double *X, const double *W, double *Phi,
                           long B, long H, long N, long Din, long C) {
  const double sc = 1.0 / sqrt((double)C);
#pragma omp parallel for schedule(static)
  for (long r = 0; r < B * H * N; ++r) {
    const double *x = X + r * Din, *w = W + ((r / N) % H) * C * Din;
    double nx = 0.0;
    for (long d = 0; d < Din; ++d) nx += x[d] * x[d];
    for (long c = 0; c < C; ++c) {
      double t = 0.0;
      for (long d = 0; d < Din; ++d) t += w[c * Din + d] * x[d];
      Phi[r * C + c] = exp(t - 0.5 * nx) * sc;
    }
  }
}

/* Vector-Jacobian product of orc_feature_performer: d phi_c / d x =
 * phi_c (w_c - x), so dX = sum_c dPhi_c phi_c (w_c - x). */
void orc_feature_performer_vjp(const double *X, const double *W,
                               const double *dPhi, double *dX, long B, long H,
                               long N, long Din, long C) {
  const double sc = 1.0 / sqrt((double)C);
#pragma omp parallel for schedule(static)
  for (long r = 0; r < B * H * N; ++r) {
    const double *x = X + r * Din, *w = W + ((r / N) % H) * C * Din;
    double nx = 0.0;
    for (long d = 0; d < Din; ++d) nx += x[d] * x[d];
    for (long d = 0; d < Din; ++d) dX[r * Din + d] = 0.0;
    for (long c = 0; c < C; ++c) {
      double t = 0.0;
      for (long d = 0; d < Din; ++d) t += w[c * Din + d] * x[d];
      const double gphi = dPhi[r * C + c] * exp(t - 0.5 * nx) * sc;
      for (long d = 0; d < Din; ++d) dX[r * Din + d] += gphi * (w[c * Din + d] - x[d]);
    }
  }
}

/*
 * Degree-2 polynomial features ("Linear Attention/zh", feature maps:
 * phi(x) = (1, x, x (x) x, ...) truncated; "Transformers are RNNs -- part
 * 2/3", section 3.2.1: the polynomial kernel has an exact finite feature
 * map, degree 2 costs O(N D^2 M)):
 *   phi(x) = (1, x_1 .. x_Din, x_a x_b for a, b = 1..Din, a-major),
 * followed by zeros up to C >= 1 + Din + Din^2, so that
 * phi(x) . phi(y) = 1 + x . y + (x . y)^2.  X [rows, Din], Phi [rows, C].
 */
void orc_feature_poly2(const double *X, double *Phi, long rows, long Din,
                       long C) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    const double *x = X + r * Din;
    double *f = Phi + r * C;
    for (long c = 0; c < C; ++c) f[c] = 0.0;
    f[0] = 1.0;
    for (long a = 0; a < Din; ++a) f[1 + a] = x[a];
    for (long a = 0; a < Din; ++a)
      for (long b = 0; b < Din; ++b) f[1 + Din + a * Din + b] = x[a] * x[b];
  }
}

/* Vector-Jacobian product of orc_feature_poly2: dX_a = dPhi[1 + a] +
 * sum_b (dPhi[1 + Din + a Din + b] + dPhi[1 + Din + b Din + a]) x_b. */
void orc_feature_poly2_vjp(const double *X, const double *dPhi, double *dX,
                           long rows, long Din, long C) {
#pragma omp parallel for schedule(static)
  for (long r = 0; r < rows; ++r) {
    const double *x = X + r * Din, *g = dPhi + r * C;
    for (long a = 0; a < Din; ++a) {
      double acc = g[1 + a];
      for (long b = 0; b < Din; ++b)
        acc += (g[1 + Din + a * Din + b] + g[1 + Din + b * Din + a]) * x[b];
      dX[r * Din + a] = acc;
    }
  }
}

/* Threads the OpenMP runtime will use (1 when built without OpenMP). */
int orc_num_threads(void) {
#ifdef _OPENMP
  extern int omp_get_max_threads(void);
  return omp_get_max_threads();
#else
  return 1;
#endif
}
