/*
 * kda_oracle.c -- fp64 CPU oracle of the KDA recurrence.
 *
 * TEST INFRASTRUCTURE ONLY: the reference the GPU path is checked against.
 * Only tests/, the smoke entry point and the benchmark's CPU-baseline leg may
 * load it.  It shares no code with the GPU path.  See kda_oracle.h for the
 * definition, layouts and citations.
 *
 * Plain token loop, exactly in the order the GLM-5.3-Flash model notes print
 * the gated delta rule (decay, read-back on the decayed state, scaled error,
 * rank-1 update); the output line, which the snippet does not print, reads the
 * state after the update, o_t = scale * S_t^T q_t.  No blocking, no fusion, no
 * reordering: one (unit, token) at a time, fp64 throughout, libm exp().
 * Units (sequence or document, head) are independent and run in parallel
 * under OpenMP, longest first.
 *
 * Build: gcc -O2 -fopenmp -fPIC -shared (no -ffast-math).
 */
#include "kda_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

typedef struct {
  int64_t n;     /* sequence / document index */
  int64_t h;     /* head */
  int64_t start; /* first token (flattened row index) */
  int64_t len;   /* number of tokens */
} unit_t;

static int by_len_desc(const void* a, const void* b) {
  const unit_t* x = (const unit_t*)a;
  const unit_t* y = (const unit_t*)b;
  if (x->len != y->len) return x->len < y->len ? 1 : -1;
  if (x->n != y->n) return x->n < y->n ? -1 : 1;
  return x->h < y->h ? -1 : (x->h > y->h);
}

/* One unit: the token loop of the gated delta rule. S is dk x dv, row i =
 * key channel i, column j = value channel j. */
static void run_unit(const unit_t* u, int64_t H, int64_t dk, int64_t dv,
                     const double* q, const double* k, const double* v,
                     const double* log_g, const double* beta,
                     const double* init_state, double scale, double* out,
                     double* final_state, double* S, double* kv, double* delta) {
  const int64_t n = u->n, h = u->h;
  if (init_state)
    memcpy(S, init_state + (n * H + h) * dk * dv, sizeof(double) * dk * dv);
  else
    memset(S, 0, sizeof(double) * dk * dv);

  for (int64_t t = u->start; t < u->start + u->len; ++t) {
    const double* kt = k + (t * H + h) * dk;
    const double* qt = q + (t * H + h) * dk;
    const double* gt = log_g + (t * H + h) * dk;
    const double* vt = v + (t * H + h) * dv;
    const double bt = beta[t * H + h];
    double* ot = out + (t * H + h) * dv;

    /* decay: every key channel i of the state by its own gate exp(log_g) */
    for (int64_t i = 0; i < dk; ++i) {
      const double a = exp(gt[i]);
      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= a;
    }
    /* read back the decayed state's prediction for k_t: kv = S^T k_t */
    for (int64_t j = 0; j < dv; ++j) kv[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) kv[j] += S[i * dv + j] * kt[i];
    /* beta-scaled prediction error */
    for (int64_t j = 0; j < dv; ++j) delta[j] = bt * (vt[j] - kv[j]);
    /* rank-1 update S += k_t delta^T */
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += kt[i] * delta[j];
    /* output from the updated state: o_t = scale * S_t^T q_t */
    for (int64_t j = 0; j < dv; ++j) {
      double acc = 0.0;
      for (int64_t i = 0; i < dk; ++i) acc += S[i * dv + j] * qt[i];
      ot[j] = scale * acc;
    }
  }
  if (final_state)
    memcpy(final_state + (n * H + h) * dk * dv, S, sizeof(double) * dk * dv);
}

int kda_oracle_threads(int n_threads) {
#ifdef _OPENMP
  return n_threads > 0 ? n_threads : omp_get_max_threads();
#else
  (void)n_threads;
  return 1;
#endif
}

int kda_oracle_forward(int64_t num_seqs, int64_t seq_len, int64_t num_heads,
                       int64_t dk, int64_t dv, const double* q, const double* k,
                       const double* v, const double* log_g, const double* beta,
                       const double* init_state, const int64_t* cu_seqlens,
                       double scale, double* out, double* final_state,
                       int n_threads) {
  if (!q || !k || !v || !log_g || !beta || !out) return -1;
  if (num_seqs < 0 || seq_len < 0 || num_heads <= 0 || dk <= 0 || dv <= 0)
    return -2;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != seq_len) return -3;
    for (int64_t n = 0; n < num_seqs; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -3;
  }

  const int64_t n_units = num_seqs * num_heads;
  unit_t* units = (unit_t*)malloc(sizeof(unit_t) * (n_units > 0 ? n_units : 1));
  if (!units) return -4;
  for (int64_t n = 0; n < num_seqs; ++n) {
    const int64_t start = cu_seqlens ? cu_seqlens[n] : n * seq_len;
    const int64_t len = cu_seqlens ? cu_seqlens[n + 1] - cu_seqlens[n] : seq_len;
    for (int64_t h = 0; h < num_heads; ++h) {
      unit_t* u = &units[n * num_heads + h];
      u->n = n;
      u->h = h;
      u->start = start;
      u->len = len;
    }
  }
  qsort(units, (size_t)n_units, sizeof(unit_t), by_len_desc);

  int failed = 0;
#ifdef _OPENMP
  const int nt = kda_oracle_threads(n_threads);
#pragma omp parallel num_threads(nt)
#endif
  {
    double* S = (double*)malloc(sizeof(double) * (dk * dv + 2 * dv));
    if (!S) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    }
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
    for (int64_t u = 0; u < n_units; ++u) {
      if (!S) continue;
      run_unit(&units[u], num_heads, dk, dv, q, k, v, log_g, beta, init_state,
               scale, out, final_state, S, S + dk * dv, S + dk * dv + dv);
    }
    free(S);
  }
  free(units);
  return failed ? -4 : 0;
}
