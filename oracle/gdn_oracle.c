/*
 * gdn_oracle.c -- fp64 token-serial CPU oracle for the gated delta rule.
 *
 * TEST INFRASTRUCTURE ONLY (see gdn_oracle.h for who may load it and what it
 * computes).  Plain C99 + OpenMP, no BLAS, no code shared with the HIP path.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

int gdn_oracle_max_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* One (sequence, value head) chain, evaluated token by token. */
static void run_unit(int64_t t0, int64_t t1, int hk, int hv, int h, int kh, int dk, int dv,
                     int per_channel, const double* q, const double* k, const double* v,
                     const double* g, const double* beta, const double* h0_unit, double* o,
                     double* hT_unit, int mutant, double* H, double* w, double* u, double* dec) {
  const size_t nstate = (size_t)dk * dv;
  if (h0_unit)
    memcpy(H, h0_unit, nstate * sizeof(double));
  else
    memset(H, 0, nstate * sizeof(double));

  for (int64_t t = t0; t < t1; ++t) {
    const double* kt = k + ((size_t)t * hk + kh) * dk;
    const double* qt = q + ((size_t)t * hk + kh) * dk;
    const double* vt = v + ((size_t)t * hv + h) * dv;
    const double bt = beta[(size_t)t * hv + h];

    /* gate of this token (natural log); the planted off-by-one mistake reads
     * the next token's gate instead */
    int64_t tg = t;
    if (mutant == GDN_ORACLE_MUT_GATE_NEXT_TOKEN && t + 1 < t1) tg = t + 1;
    if (per_channel) {
      const double* gt = g + ((size_t)tg * hv + h) * dk;
      for (int c = 0; c < dk; ++c) dec[c] = exp(gt[c]);
    } else {
      const double a = exp(g[(size_t)tg * hv + h]);
      for (int c = 0; c < dk; ++c) dec[c] = a;
    }

    /* 1. decay: H <- D_t H (row c of the K-first state scales by dec[c]) */
    if (mutant != GDN_ORACLE_MUT_DECAY_AFTER_WRITE) {
      for (int c = 0; c < dk; ++c) {
        double* row = H + (size_t)c * dv;
        for (int j = 0; j < dv; ++j) row[j] *= dec[c];
      }
    }

    /* planted mistake: read the output before this token's write */
    if (mutant == GDN_ORACLE_MUT_OUTPUT_BEFORE_WRITE && o) {
      double* ot = o + ((size_t)t * hv + h) * dv;
      for (int j = 0; j < dv; ++j) ot[j] = 0.0;
      for (int c = 0; c < dk; ++c) {
        const double* row = H + (size_t)c * dv;
        for (int j = 0; j < dv; ++j) ot[j] += row[j] * qt[c];
      }
    }

    /* 2. w = H^T k ;  u = beta (v - w) */
    for (int j = 0; j < dv; ++j) w[j] = 0.0;
    for (int c = 0; c < dk; ++c) {
      const double* row = H + (size_t)c * dv;
      const double kc = kt[c];
      for (int j = 0; j < dv; ++j) w[j] += row[j] * kc;
    }
    if (mutant == GDN_ORACLE_MUT_NO_BETA_ERASE) {
      for (int j = 0; j < dv; ++j) u[j] = bt * vt[j] - w[j];
    } else {
      for (int j = 0; j < dv; ++j) u[j] = bt * (vt[j] - w[j]);
    }

    /* 3. H <- H + k u^T */
    for (int c = 0; c < dk; ++c) {
      double* row = H + (size_t)c * dv;
      const double kc = kt[c];
      for (int j = 0; j < dv; ++j) row[j] += kc * u[j];
    }
    if (mutant == GDN_ORACLE_MUT_DECAY_AFTER_WRITE) {
      for (int c = 0; c < dk; ++c) {
        double* row = H + (size_t)c * dv;
        for (int j = 0; j < dv; ++j) row[j] *= dec[c];
      }
    }

    /* 4. o_t = H^T q  (the planted transposed read uses H q instead) */
    if (o && mutant != GDN_ORACLE_MUT_OUTPUT_BEFORE_WRITE) {
      double* ot = o + ((size_t)t * hv + h) * dv;
      if (mutant == GDN_ORACLE_MUT_TRANSPOSED_READ && dk == dv) {
        for (int r = 0; r < dk; ++r) {
          const double* row = H + (size_t)r * dv;
          double s = 0.0;
          for (int j = 0; j < dv; ++j) s += row[j] * qt[j];
          ot[r] = s;
        }
      } else {
        for (int j = 0; j < dv; ++j) ot[j] = 0.0;
        for (int c = 0; c < dk; ++c) {
          const double* row = H + (size_t)c * dv;
          const double qc = qt[c];
          for (int j = 0; j < dv; ++j) ot[j] += row[j] * qc;
        }
      }
    }
  }
  if (hT_unit) memcpy(hT_unit, H, nstate * sizeof(double));
}

int gdn_oracle_fwd(int n_seq, const int64_t* seq_start, int hk, int hv, const int32_t* head_map,
                   int dk, int dv, int per_channel, const double* q, const double* k, const double* v,
                   const double* g, const double* beta, const double* h0, double* o, double* hT,
                   const int32_t* units, int n_units, int n_threads, int mutant) {
  if (n_seq < 0 || hk <= 0 || hv <= 0 || dk <= 0 || dv <= 0) return -1;
  if (!seq_start) return -2;
  if (!head_map && hv % hk != 0) return -3;
  for (int n = 0; n < n_seq; ++n)
    if (seq_start[n + 1] < seq_start[n]) return -4;
  if (head_map)
    for (int h = 0; h < hv; ++h)
      if (head_map[h] < 0 || head_map[h] >= hk) return -5;
  const int group = head_map ? 1 : hv / hk;
  const long total_units = units ? (long)n_units : (long)n_seq * hv;
  if (units)
    for (long i = 0; i < total_units; ++i)
      if (units[2 * i] < 0 || units[2 * i] >= n_seq || units[2 * i + 1] < 0 || units[2 * i + 1] >= hv)
        return -6;
  const size_t nstate = (size_t)dk * dv;

#ifdef _OPENMP
  if (n_threads > 0) omp_set_num_threads(n_threads);
#else
  (void)n_threads;
#endif

  int failed = 0;
#pragma omp parallel
  {
    double* H = (double*)malloc(nstate * sizeof(double));
    double* w = (double*)malloc((size_t)dv * sizeof(double));
    double* u = (double*)malloc((size_t)dv * sizeof(double));
    double* dec = (double*)malloc((size_t)dk * sizeof(double));
    if (!H || !w || !u || !dec) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (long i = 0; i < total_units; ++i) {
        const int n = units ? units[2 * i] : (int)(i / hv);
        const int h = units ? units[2 * i + 1] : (int)(i % hv);
        const int kh = head_map ? head_map[h] : h / group;
        const double* h0u = h0 ? h0 + ((size_t)n * hv + h) * nstate : NULL;
        double* hTu = hT ? hT + ((size_t)n * hv + h) * nstate : NULL;
        run_unit(seq_start[n], seq_start[n + 1], hk, hv, h, kh, dk, dv, per_channel, q, k, v, g,
                 beta, h0u, o, hTu, mutant, H, w, u, dec);
      }
    }
    free(H);
    free(w);
    free(u);
    free(dec);
  }
  return failed ? -7 : 0;
}
