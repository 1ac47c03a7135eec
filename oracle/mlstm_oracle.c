/*
 * mLSTM matrix-memory cell: plain fp64 CPU oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header or constant with the
 * HIP library.
 *
 * Source of the method (cited by page title and section):
 *   [xLSTM-post] "xLSTM: How Exponential Gating and Matrix Memory Scale
 *   Recurrent Neural Networks" (llms.blog), section 3 "mLSTM: Matrix Memory
 *   and the Parallel Dual Form", sub-section "Associative Matrix Cell State"
 *   (the update of C, the update of n, the retrieval h~ and h = o (.) h~), and
 *   section 2, sub-section "The Normalizer State and Numerical Stabilization"
 *   (the running maximum m and the two stabilized update factors).
 *
 * What is computed, per (batch b, head h), token by token in order:
 *
 *   log f_t = logsigmoid(f~_t)   (sigmoid forget gate)   or   f~_t (exp gate)
 *   m_t     = max(log f_t + m_{t-1}, i~_t)                 running maximum
 *   fp      = exp(log f_t + m_{t-1} - m_t)                 stabilized f_t
 *   ip      = exp(i~_t - m_t)                              stabilized i_t
 *   C~_t    = fp * C~_{t-1} + ip * k_t v_t^T      (stored [d_qk][d_v])
 *   n~_t    = fp * n~_{t-1} + ip * k_t
 *   num_t   = q_t^T C~_t                          (length d_v)
 *   den_t   = max(|n~_t . q_t|, exp(-m_t))
 *   h_t     = sigmoid(o~_t) (.) num_t / den_t     (o~ absent: gate = 1)
 *
 * Readings of the pages taken here (each is listed in the design notes):
 *  - The state is carried in stabilized form (C~, n~, m): the true memory is
 *    C = C~ e^m and n = n~ e^m.  With this, max(|n~.q|, e^{-m}) equals
 *    e^{-m} max(|n.q|, 1), i.e. the page's retrieval denominator
 *    max(n^T q, 1) with an absolute value, and the common e^{-m} cancels.
 *  - The page writes C as the sum of v k^T (d_v x d_qk).  It is stored here
 *    transposed, [d_qk][d_v], so the readout is q^T C~; the numbers are the
 *    same.
 *  - k arrives already scaled by 1/sqrt(d_qk) (the page folds that factor into
 *    the definition of k); q is unscaled.
 *  - The readout at token t uses the memory after token t's own update.
 *  - A missing initial state means C~ = 0, n~ = 0, m = 0.
 *
 * All sums run in ascending index order.  No blocking, no reordering.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_FGATE_SIGMOID 0
#define ORACLE_FGATE_EXP 1

static double logsigmoid(double x) {
  /* log(1 / (1 + e^{-x})) written without overflow */
  double a = x < 0.0 ? x : 0.0;
  return a - log1p(exp(-fabs(x)));
}

static double sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double dmax(double a, double b) { return a > b ? a : b; }

/*
 * One token of the recurrence for one head.  State (C, n, *m) is updated in
 * place; h (length dv) receives the output.  o may be NULL (gate = 1).
 */
static void oracle_token(int64_t dqk, int64_t dv, int fgate,
                         const double* q, const double* k, const double* v,
                         double i_pre, double f_pre, const double* o,
                         double* C, double* n, double* m, double* h) {
  double lf = (fgate == ORACLE_FGATE_SIGMOID) ? logsigmoid(f_pre) : f_pre;
  double m_new = dmax(lf + *m, i_pre);
  double fp = exp(lf + *m - m_new);
  double ip = exp(i_pre - m_new);
  for (int64_t a = 0; a < dqk; ++a) {
    double ika = ip * k[a];
    double* row = C + a * dv;
    for (int64_t b = 0; b < dv; ++b) row[b] = fp * row[b] + ika * v[b];
    n[a] = fp * n[a] + ika;
  }
  *m = m_new;
  double nq = 0.0;
  for (int64_t a = 0; a < dqk; ++a) nq += n[a] * q[a];
  double den = dmax(fabs(nq), exp(-m_new));
  for (int64_t b = 0; b < dv; ++b) {
    double num = 0.0;
    for (int64_t a = 0; a < dqk; ++a) num += q[a] * C[a * dv + b];
    double gate = o ? sigmoid(o[b]) : 1.0;
    h[b] = gate * num / den;
  }
}

static void set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
}

/* Number of threads OpenMP will use for the next parallel region. */
int oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/*
 * Full sequence, all heads.  Layouts (row-major, contiguous):
 *   q, k [B,H,T,dqk]; v, o, h [B,H,T,dv]; i_pre, f_pre [B,H,T];
 *   C0, C1 [B,H,dqk,dv]; n0, n1 [B,H,dqk]; m0, m1 [B,H].
 * o, C0, n0, m0 may be NULL (o = 1; zero state).  C1, n1, m1 may be NULL.
 * Heads are independent, so they are spread over threads; within a head
 * the tokens are processed strictly in order.
 */
void oracle_recurrent(int64_t B, int64_t H, int64_t T, int64_t dqk, int64_t dv,
                      int fgate, const double* q, const double* k,
                      const double* v, const double* i_pre,
                      const double* f_pre, const double* o, const double* C0,
                      const double* n0, const double* m0, double* h,
                      double* C1, double* n1, double* m1, int nthreads) {
  set_threads(nthreads);
  int64_t BH = B * H;
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < BH; ++bh) {
    double* C = (double*)malloc(sizeof(double) * (size_t)(dqk * dv + dqk));
    double* n = C + dqk * dv;
    double m = 0.0;
    if (C0) {
      memcpy(C, C0 + bh * dqk * dv, sizeof(double) * (size_t)(dqk * dv));
      memcpy(n, n0 + bh * dqk, sizeof(double) * (size_t)dqk);
      m = m0[bh];
    } else {
      memset(C, 0, sizeof(double) * (size_t)(dqk * dv + dqk));
    }
    for (int64_t t = 0; t < T; ++t) {
      int64_t tok = bh * T + t;
      oracle_token(dqk, dv, fgate, q + tok * dqk, k + tok * dqk, v + tok * dv,
                   i_pre[tok], f_pre[tok], o ? o + tok * dv : NULL, C, n, &m,
                   h + tok * dv);
    }
    if (C1) memcpy(C1 + bh * dqk * dv, C, sizeof(double) * (size_t)(dqk * dv));
    if (n1) memcpy(n1 + bh * dqk, n, sizeof(double) * (size_t)dqk);
    if (m1) m1[bh] = m;
    free(C);
  }
}

/*
 * One token for every head (the decode step).  Layouts:
 *   q, k [B,H,dqk]; v, o, h [B,H,dv]; i_pre, f_pre [B,H];
 *   C [B,H,dqk,dv], n [B,H,dqk], m [B,H] are read and overwritten in place.
 */
void oracle_step(int64_t B, int64_t H, int64_t dqk, int64_t dv, int fgate,
                 const double* q, const double* k, const double* v,
                 const double* i_pre, const double* f_pre, const double* o,
                 double* C, double* n, double* m, double* h, int nthreads) {
  set_threads(nthreads);
  int64_t BH = B * H;
#pragma omp parallel for schedule(static)
  for (int64_t bh = 0; bh < BH; ++bh) {
    oracle_token(dqk, dv, fgate, q + bh * dqk, k + bh * dqk, v + bh * dv,
                 i_pre[bh], f_pre[bh], o ? o + bh * dv : NULL,
                 C + bh * dqk * dv, n + bh * dqk, m + bh, h + bh * dv);
  }
}
