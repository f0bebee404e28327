/*
 * streamkl_oracle.c -- plain fp64 CPU oracle for the attention-KL divergence
 * and its gradients.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the yardstick the GPU library is
 * checked against; it is not part of the product path.  Only the tests, the
 * smoke check and the benchmark's CPU-baseline leg may load it.  It shares no
 * code, header, table or helper with the HIP library.
 *
 * What it computes follows the StreamKL summary page (gist.science, paper
 * 2606.20005), written the slow, obvious way: the N_Q x N_K score and
 * probability rows ARE materialised here (one query row at a time), which is
 * exactly the "materialising" computation the page's Problem section
 * describes and the fused method replaces.  No online recurrence is used.
 *
 * Per attention head (b, h) and query row i, in double precision:
 *   J_i       allowed keys: all j < N_K, or, when causal, j <= i + (N_K - N_Q)
 *             (causal mask aligned bottom-right; equals j <= i for square
 *             problems -- a reading, the page does not fix the alignment).
 *   S_t[i,j]  = scale * <q_t[i], k_t[j]>                  (t = 1 teacher, 2 student)
 *   LSE_t[i]  = log sum_{j in J_i} exp(S_t[i,j])   (max-shifted, two passes)
 *             -- "Formulazione Online" section, LSE_t = m_t + log l_t.
 *   logP_t    = S_t - LSE_t ;  P_t = exp(logP_t)
 *             -- "Strategia di Ricalcolo" section, P = exp(S - LSE); the
 *             log-ratio is formed from logits and LSEs, never from log(P)
 *             ("Stabilita Numerica" bullet of the kernel-optimisation section).
 *   KL[i]     = sum_j P1 (logP1 - logP2)          -- KL(P1 || P2) by definition
 *             (Problem section); the page's L = acc/l1 + LSE2 - LSE1 is the
 *             same quantity, rearranged.
 *   g[i]      upstream gradient of the per-row KL (NULL means all ones).
 *   dS2[i,j]  = g[i] (P2 - P1)                    -- Configuration 1 (P1 fixed)
 *   dS1[i,j]  = g[i] P1 (logP1 - logP2 - KL[i])   -- Configuration 2 (P2 fixed)
 *             Both are zero outside J_i.  These are the partial derivatives of
 *             KL[i] with respect to the scaled logits; the page names the two
 *             configurations but prints neither formula.
 *   dQ_t[i]   = scale * sum_j dS_t[i,j] k_t[j]
 *   dK_t[j]  += scale * sum_i dS_t[i,j] q_t[i]
 *
 * Layout: every tensor is a dense row-major [rows, d] slab per head, heads
 * contiguous ([B, H, N, d] with d innermost); per-row vectors are [B, H, N_Q].
 */
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

static double dot(const double *a, const double *b, int d) {
  double s = 0.0;
  for (int c = 0; c < d; ++c) s += a[c] * b[c];
  return s;
}

/* Number of allowed keys for query row i. */
static int allowed_keys(int i, int n_q, int n_k, int causal) {
  if (!causal) return n_k;
  int last = i + (n_k - n_q); /* last allowed key index */
  if (last < 0) return 0;
  return last + 1 < n_k ? last + 1 : n_k;
}

/* log-sum-exp of x[0..n) with the maximum shifted out. */
static double logsumexp(const double *x, int n) {
  double m = -INFINITY;
  for (int j = 0; j < n; ++j)
    if (x[j] > m) m = x[j];
  double s = 0.0;
  for (int j = 0; j < n; ++j) s += exp(x[j] - m);
  return m + log(s);
}

/*
 * One query row of one head.  s1, s2 are caller scratch of n_k doubles.
 * Writes kl/lse1/lse2 for the row; if dq1 != NULL also writes the row's dq1,
 * dq2 and adds its contribution into dk1, dk2 (which must then be non-NULL).
 */
static void one_row(const double *q1, const double *k1, const double *q2,
                    const double *k2, int n_q, int n_k, int d, double scale,
                    int causal, int i, double g, double *s1, double *s2,
                    double *kl, double *lse1, double *lse2, double *dq1,
                    double *dk1, double *dq2, double *dk2) {
  const int nj = allowed_keys(i, n_q, n_k, causal);
  const double *qi1 = q1 + (size_t)i * d;
  const double *qi2 = q2 + (size_t)i * d;

  for (int j = 0; j < nj; ++j) {
    s1[j] = scale * dot(qi1, k1 + (size_t)j * d, d);
    s2[j] = scale * dot(qi2, k2 + (size_t)j * d, d);
  }
  const double L1 = logsumexp(s1, nj);
  const double L2 = logsumexp(s2, nj);

  double klv = 0.0;
  for (int j = 0; j < nj; ++j) {
    double lp1 = s1[j] - L1, lp2 = s2[j] - L2;
    klv += exp(lp1) * (lp1 - lp2);
  }
  kl[i] = klv;
  lse1[i] = L1;
  lse2[i] = L2;
  if (!dq1) return;

  double *gq1 = dq1 + (size_t)i * d;
  double *gq2 = dq2 + (size_t)i * d;
  for (int c = 0; c < d; ++c) gq1[c] = gq2[c] = 0.0;
  for (int j = 0; j < nj; ++j) {
    double lp1 = s1[j] - L1, lp2 = s2[j] - L2;
    double p1 = exp(lp1), p2 = exp(lp2);
    double ds2 = g * (p2 - p1);
    double ds1 = g * p1 * (lp1 - lp2 - klv);
    const double *kj1 = k1 + (size_t)j * d;
    const double *kj2 = k2 + (size_t)j * d;
    double *gk1 = dk1 + (size_t)j * d;
    double *gk2 = dk2 + (size_t)j * d;
    for (int c = 0; c < d; ++c) {
      gq1[c] += scale * ds1 * kj1[c];
      gq2[c] += scale * ds2 * kj2[c];
      gk1[c] += scale * ds1 * qi1[c];
      gk2[c] += scale * ds2 * qi2[c];
    }
  }
}

/*
 * oracle_head: rows [row_begin, row_end) of one head.
 *   Inputs  q1, q2: [n_q, d]; k1, k2: [n_k, d]; g: [n_q] or NULL (ones).
 *   Outputs kl, lse1, lse2: [n_q] (only the rows in range are written).
 *   If dq1 is non-NULL: dq1, dq2 [n_q, d] rows in range are overwritten and
 *   dk1, dk2 [n_k, d] are fully overwritten with the contribution of the rows
 *   in range (the whole gradient when the range is [0, n_q)).
 * Rows are split over OpenMP threads; key gradients use per-thread partial
 * sums that are added up at the end.
 * Returns 0, or -1 if scratch memory cannot be allocated.
 */
int oracle_head(const double *q1, const double *k1, const double *q2,
                const double *k2, const double *g, int n_q, int n_k, int d,
                double scale, int causal, int row_begin, int row_end,
                double *kl, double *lse1, double *lse2, double *dq1,
                double *dk1, double *dq2, double *dk2) {
  const int want_grad = dq1 != NULL;
  const size_t kd = (size_t)n_k * d;
  if (want_grad) {
    memset(dk1, 0, kd * sizeof(double));
    memset(dk2, 0, kd * sizeof(double));
  }
  int failed = 0;
#pragma omp parallel
  {
    double *s1 = (double *)malloc(sizeof(double) * (n_k > 0 ? n_k : 1));
    double *s2 = (double *)malloc(sizeof(double) * (n_k > 0 ? n_k : 1));
    double *pk1 = NULL, *pk2 = NULL;
    if (want_grad) {
      pk1 = (double *)calloc(kd > 0 ? kd : 1, sizeof(double));
      pk2 = (double *)calloc(kd > 0 ? kd : 1, sizeof(double));
    }
    int ok = s1 && s2 && (!want_grad || (pk1 && pk2));
    if (!ok) {
#pragma omp atomic write
      failed = 1;
    }
#pragma omp for schedule(dynamic, 4)
    for (int i = row_begin; i < row_end; ++i) {
      if (!ok) continue;
      double gi = g ? g[i] : 1.0;
      one_row(q1, k1, q2, k2, n_q, n_k, d, scale, causal, i, gi, s1, s2, kl,
              lse1, lse2, dq1, pk1, dq2, pk2);
    }
    if (want_grad && ok) {
#pragma omp critical
      {
        for (size_t u = 0; u < kd; ++u) {
          dk1[u] += pk1[u];
          dk2[u] += pk2[u];
        }
      }
    }
    free(s1);
    free(s2);
    free(pk1);
    free(pk2);
  }
  return failed ? -1 : 0;
}

/* Threads the OpenMP runtime will use for the next parallel region. */
int oracle_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}
