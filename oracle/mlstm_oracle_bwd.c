/*
 * mLSTM matrix-memory cell: plain fp64 CPU oracle of the gradient of the
 * forward pass (reverse mode through the token recurrence).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or
 * call this file; only the test suite uses it.  It shares no code, header or
 * constant with the HIP library (nor with mlstm_oracle.c: it is written out
 * on its own).
 *
 * Source of the method (cited by page title and section):
 *   [xLSTM-post] "xLSTM: How Exponential Gating and Matrix Memory Scale
 *   Recurrent Neural Networks" (llms.blog), section 3, sub-section
 *   "Associative Matrix Cell State": C_t = f_t C_{t-1} + i_t v_t k_t^T,
 *   n_t = f_t n_{t-1} + i_t k_t, h~_t = C_t q_t / max(n_t^T q_t, 1),
 *   h_t = o_t (.) h~_t; the gates of section 2 (i_t = exp(i~_t), f_t =
 *   sigmoid(f~_t) or exp(f~_t)).  The pages motivate the parallel form by
 *   training; they print no gradient, so this file differentiates the
 *   recurrence directly.
 *
 * What is computed, per (batch b, head h).  The recurrence is run in true
 * (unstabilized) units, which fp64 holds for the supported range |m| <= 80:
 *
 *   C_0 = C~0 e^{m0}, n_0 = n~0 e^{m0}              (zero when absent)
 *   C_t = f_t C_{t-1} + i_t k_t v_t^T  ([d_qk][d_v]), n_t = f_t n_{t-1} + i_t k_t
 *   num_t = q_t^T C_t, nq_t = n_t . q_t, den_t = max(|nq_t|, 1)
 *   h_t = sigmoid(o~_t) (.) num_t / den_t           (o~ absent: gate 1)
 *
 * (the forward oracle's stabilized recurrence gives the same h: there the
 * denominator is e^{-m_t} max(|nq_t|, 1)).  The scalar whose gradient is
 * returned is
 *
 *   L = sum_t dh_t . h_t + e^{-m_T} (<dC1, C_T> + <dn1, n_T>)
 *
 * where m_T is the final running maximum (held constant): dC1 and dn1 are
 * the gradients of a loss with respect to the final memory, given in the
 * scale of the stored final state C~_T = C_T e^{-m_T}.  In the same way the
 * gradients of the initial state are returned in its stored scale:
 * dC~0 = e^{m0} dL/dC_0, dn~0 = e^{m0} dL/dn_0, and
 * dm0 = <dL/dC_0, C_0> + <dL/dn_0, n_0> (the derivative through the factor
 * e^{m0} of the true initial memory).
 *
 * Reverse step at token t (GC, Gn: dL/dC_t, dL/dn_t accumulated so far):
 *   h_t = gate (.) num / den_t (or the given h_in, below)
 *   dnum = gate (.) dh_t / den_t,  dden = -(dh_t . h_t) / den_t
 *   dnq  = dden * sign(nq_t) where |nq_t| >= 1, else 0
 *   GC += q_t dnum^T,  Gn += dnq q_t
 *   dq_t = C_t dnum + dnq n_t
 *   do~_t = dh_t (.) h_t (.) (1 - gate)
 *   dk_t = i_t (GC v_t + Gn),  dv_t = i_t GC^T k_t
 *   di~_t = i_t (k_t^T GC v_t + k_t . Gn)
 *   df~_t = (<GC, C_{t-1}> + <Gn, n_{t-1}>) * df_t/df~_t
 *           (f (1 - f) for the sigmoid gate, f for the exp gate)
 *   GC <- f_t GC,  Gn <- f_t Gn
 *
 * The states C_{t-1} of the reverse sweep are recomputed segment by segment
 * (SEG tokens) from checkpoints taken in the forward sweep.  Sums run in
 * ascending index order.
 *
 * Given forward output (h_in).  A backward pass that is handed the forward
 * output h uses it where the gradient depends on h itself: the denominator
 * term, dden = -(dh_t . h_t) / den_t, and do~_t = dh_t (.) h_t (.) (1 - gate).
 * With h_in = NULL these use the oracle's own fp64 h (num/den above, the
 * same value).  With h_in set (e.g. the fp64 h rounded to bfloat16, as a
 * bf16 forward pass hands it over) the result is that same formula
 * evaluated at the given h, so two implementations handed the same h can be
 * compared without the rounding of h in between.
 *
 * Conditioning (cond_dq, cond_dk, cond_di, cond_df, cond_dm0).  These five
 * gradients are each the sum of a memory path and a normalizer path:
 *   dq_t   = C_t dnum + dnq n_t,
 *   dk_t   = i_t (GC v_t + Gn),
 *   di~_t  = i_t (k_t^T GC v_t + k_t . Gn),
 *   df~_t  = (<GC, C_{t-1}> + <Gn, n_{t-1}>) df_t/df~_t,
 *   dm0    = <GC, C_0> + <Gn, n_0>.
 * On the active branch of the denominator (|n.q| >= 1) the readout does not
 * change when q is scaled, nor when C and n are scaled together, so the two
 * paths partly cancel.  The returned cond = the same sums with each path's
 * absolute value (elementwise for dq, dk):
 *   |C_t dnum| + |dnq n_t|,  i_t (|GC v_t| + |Gn|),
 *   i_t (|k_t^T GC v_t| + |k_t . Gn|),
 *   (|<GC, C_{t-1}>| + |<Gn, n_{t-1}>|) |df_t/df~_t|,  |<GC, C_0>| + |<Gn, n_0>|,
 * is the scale against which an error made in the paths is measured: a
 * relative error e in the paths gives an error of about e cond in the sum,
 * however small the sum itself is.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define BWD_FGATE_SIGMOID 0
#define SEG 64

static double bwd_sigmoid(double x) { return 1.0 / (1.0 + exp(-x)); }

static double bwd_log_forget(double f_pre, int fgate) {
  if (fgate == BWD_FGATE_SIGMOID) {
    double a = f_pre < 0.0 ? f_pre : 0.0;
    return a - log1p(exp(-fabs(f_pre)));
  }
  return f_pre;
}

/* One forward token in true units: C, n updated in place. */
static void bwd_update(int64_t dqk, int64_t dv, double f, double i,
                       const double* k, const double* v, double* C, double* n) {
  for (int64_t a = 0; a < dqk; ++a) {
    double ika = i * k[a];
    double* row = C + a * dv;
    for (int64_t b = 0; b < dv; ++b) row[b] = f * row[b] + ika * v[b];
    n[a] = f * n[a] + ika;
  }
}

/*
 * Layouts (row-major, contiguous): q, k, dq, dk, cond_dq, cond_dk [B,H,T,dqk];
 * v, o, dh, h_in,
 * dv_out, do_out [B,H,T,dv]; i_pre, f_pre, di, df, cond_di, cond_df [B,H,T];
 * C0, dC1, dC0 [B,H,dqk,dv]; n0, dn1, dn0 [B,H,dqk]; m0, dm0, cond_dm0
 * [B,H].  o, h_in, C0/n0/m0 (together), dC1/dn1 (together) may be NULL;
 * do_out must be non-NULL when o is; dC0, dn0, dm0 and the cond_ arrays may
 * be NULL.
 */
void oracle_backward(int64_t B, int64_t H, int64_t T, int64_t dqk, int64_t dv,
                     int fgate, const double* q, const double* k,
                     const double* v, const double* i_pre, const double* f_pre,
                     const double* o, const double* C0, const double* n0,
                     const double* m0, const double* dh, const double* h_in,
                     const double* dC1, const double* dn1, double* dq, double* dk,
                     double* dv_out, double* di, double* df, double* do_out,
                     double* dC0, double* dn0, double* dm0, double* cond_dq,
                     double* cond_dk, double* cond_di, double* cond_df,
                     double* cond_dm0, int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#else
  (void)nthreads;
#endif
  const int64_t BH = B * H;
  const int64_t nseg = (T + SEG - 1) / SEG;
  const int64_t S = dqk * dv + dqk;   /* one (C, n) pair */
#pragma omp parallel for schedule(dynamic, 1)
  for (int64_t bh = 0; bh < BH; ++bh) {
    double* ck = (double*)malloc(sizeof(double) * (size_t)((nseg + 1) * S));
    double* seg = (double*)malloc(sizeof(double) * (size_t)((SEG + 1) * S));
    double* G = (double*)malloc(sizeof(double) * (size_t)S);
    double* num = (double*)malloc(sizeof(double) * (size_t)(2 * dv));
    double* dnum = num + dv;
    double* GC = G;
    double* Gn = G + dqk * dv;
    /* ---- forward sweep: true-unit state, checkpoints, final m */
    double* C = ck;   /* checkpoint 0 = initial state */
    double scale0 = 1.0;
    if (C0) {
      scale0 = exp(m0[bh]);
      for (int64_t x = 0; x < dqk * dv; ++x) C[x] = C0[bh * dqk * dv + x] * scale0;
      for (int64_t a = 0; a < dqk; ++a) C[dqk * dv + a] = n0[bh * dqk + a] * scale0;
    } else {
      memset(C, 0, sizeof(double) * (size_t)S);
    }
    double m = C0 ? m0[bh] : 0.0;
    double* cur = seg;   /* running state */
    memcpy(cur, C, sizeof(double) * (size_t)S);
    for (int64_t t = 0; t < T; ++t) {
      const int64_t tok = bh * T + t;
      const double lf = bwd_log_forget(f_pre[tok], fgate);
      m = (lf + m > i_pre[tok]) ? lf + m : i_pre[tok];
      bwd_update(dqk, dv, exp(lf), exp(i_pre[tok]), k + tok * dqk, v + tok * dv,
                 cur, cur + dqk * dv);
      if ((t + 1) % SEG == 0) memcpy(ck + ((t + 1) / SEG) * S, cur, sizeof(double) * (size_t)S);
    }
    /* ---- reverse sweep */
    if (dC1) {
      const double s1 = exp(-m);
      for (int64_t x = 0; x < dqk * dv; ++x) GC[x] = dC1[bh * dqk * dv + x] * s1;
      for (int64_t a = 0; a < dqk; ++a) Gn[a] = dn1[bh * dqk + a] * s1;
    } else {
      memset(G, 0, sizeof(double) * (size_t)S);
    }
    for (int64_t sg = nseg - 1; sg >= 0; --sg) {
      const int64_t t0 = sg * SEG;
      const int64_t t1 = (t0 + SEG < T) ? t0 + SEG : T;
      /* seg[j] = state after token t0 + j - 1 (seg[0] = the checkpoint) */
      memcpy(seg, ck + sg * S, sizeof(double) * (size_t)S);
      for (int64_t t = t0; t < t1; ++t) {
        const int64_t tok = bh * T + t;
        double* nxt = seg + (t - t0 + 1) * S;
        memcpy(nxt, seg + (t - t0) * S, sizeof(double) * (size_t)S);
        bwd_update(dqk, dv, exp(bwd_log_forget(f_pre[tok], fgate)), exp(i_pre[tok]),
                   k + tok * dqk, v + tok * dv, nxt, nxt + dqk * dv);
      }
      for (int64_t t = t1 - 1; t >= t0; --t) {
        const int64_t tok = bh * T + t;
        const double* Ct = seg + (t - t0 + 1) * S;
        const double* nt = Ct + dqk * dv;
        const double* Cp = seg + (t - t0) * S;
        const double* np = Cp + dqk * dv;
        const double* qt = q + tok * dqk;
        const double* kt = k + tok * dqk;
        const double* vt = v + tok * dv;
        const double* dht = dh + tok * dv;
        const double f = exp(bwd_log_forget(f_pre[tok], fgate));
        const double i = exp(i_pre[tok]);
        double nq = 0.0;
        for (int64_t a = 0; a < dqk; ++a) nq += nt[a] * qt[a];
        const double den = fabs(nq) > 1.0 ? fabs(nq) : 1.0;
        double sden = 0.0;   /* sum_b dh_t[b] h_t[b] */
        for (int64_t b = 0; b < dv; ++b) {
          double acc = 0.0;
          for (int64_t a = 0; a < dqk; ++a) acc += qt[a] * Ct[a * dv + b];
          num[b] = acc;
          const double gate = o ? bwd_sigmoid(o[tok * dv + b]) : 1.0;
          const double hb = h_in ? h_in[tok * dv + b] : gate * acc / den;
          dnum[b] = gate * dht[b] / den;
          sden += dht[b] * hb;
          if (o) do_out[tok * dv + b] = dht[b] * hb * (1.0 - gate);
        }
        const double dden = -sden / den;
        const double dnq = fabs(nq) >= 1.0 ? (nq >= 0.0 ? dden : -dden) : 0.0;
        for (int64_t a = 0; a < dqk; ++a) {
          double acc = 0.0;
          for (int64_t b = 0; b < dv; ++b) {
            GC[a * dv + b] += qt[a] * dnum[b];
            acc += Ct[a * dv + b] * dnum[b];
          }
          Gn[a] += dnq * qt[a];
          dq[tok * dqk + a] = acc + dnq * nt[a];
          if (cond_dq) cond_dq[tok * dqk + a] = fabs(acc) + fabs(dnq * nt[a]);
        }
        double dI = 0.0, dF = 0.0;
        double dI_mem = 0.0, dI_nrm = 0.0, dF_mem = 0.0, dF_nrm = 0.0;   /* the two paths */
        for (int64_t a = 0; a < dqk; ++a) {
          double gv = 0.0, fc = 0.0;
          for (int64_t b = 0; b < dv; ++b) {
            gv += GC[a * dv + b] * vt[b];
            fc += GC[a * dv + b] * Cp[a * dv + b];
          }
          dk[tok * dqk + a] = i * (gv + Gn[a]);
          if (cond_dk) cond_dk[tok * dqk + a] = i * (fabs(gv) + fabs(Gn[a]));
          dI += kt[a] * (gv + Gn[a]);
          dF += fc + Gn[a] * np[a];
          dI_mem += kt[a] * gv;
          dI_nrm += kt[a] * Gn[a];
          dF_mem += fc;
          dF_nrm += Gn[a] * np[a];
        }
        for (int64_t b = 0; b < dv; ++b) {
          double acc = 0.0;
          for (int64_t a = 0; a < dqk; ++a) acc += GC[a * dv + b] * kt[a];
          dv_out[tok * dv + b] = i * acc;
        }
        const double dfdf = (fgate == BWD_FGATE_SIGMOID) ? f * (1.0 - f) : f;
        di[tok] = i * dI;
        df[tok] = dF * dfdf;
        if (cond_di) cond_di[tok] = i * (fabs(dI_mem) + fabs(dI_nrm));
        if (cond_df) cond_df[tok] = (fabs(dF_mem) + fabs(dF_nrm)) * dfdf;
        for (int64_t x = 0; x < S; ++x) G[x] *= f;
      }
    }
    /* ---- initial state, in its stored scale */
    if (dC0) for (int64_t x = 0; x < dqk * dv; ++x) dC0[bh * dqk * dv + x] = GC[x] * scale0;
    if (dn0) for (int64_t a = 0; a < dqk; ++a) dn0[bh * dqk + a] = Gn[a] * scale0;
    if (dm0 || cond_dm0) {
      double acc_mem = 0.0, acc_nrm = 0.0;
      for (int64_t x = 0; x < dqk * dv; ++x) acc_mem += G[x] * ck[x];
      for (int64_t x = dqk * dv; x < S; ++x) acc_nrm += G[x] * ck[x];
      if (dm0) dm0[bh] = acc_mem + acc_nrm;
      if (cond_dm0) cond_dm0[bh] = fabs(acc_mem) + fabs(acc_nrm);
    }
    free(ck);
    free(seg);
    free(G);
    free(num);
  }
}
