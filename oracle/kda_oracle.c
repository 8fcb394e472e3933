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

/* One unit in reverse mode.  Forward: the same token loop as run_unit, with
 * the state before every token kept in hist.  Backward: for t = last .. first,
 * dS holds dL/dS_t (the state after token t); each line below is the chain
 * rule through one line of the forward step, taken in reverse order:
 *
 *   forward step t                      reverse
 *   P = Diag(a) S_{t-1}, a = exp(g_t)    dS_{t-1} = Diag(a) dP,  dg_t[i] = a[i] sum_j dP[i,j] S_{t-1}[i,j]
 *   kv = P^T k_t                          dP += k_t dkv^T,  dk_t += P dkv
 *   delta = beta_t (v_t - kv)             dv_t = beta_t ddelta,  dkv = -beta_t ddelta,
 *                                         dbeta_t = ddelta . (v_t - kv)
 *   S_t = P + k_t delta^T                 dP = dS,  dk_t = dS delta,  ddelta = dS^T k_t
 *   o_t = scale S_t^T q_t                 dq_t = scale S_t do_t,  dS += scale q_t do_t^T
 */
static int run_unit_bwd(const unit_t* u, int64_t H, int64_t dk, int64_t dv,
                        const double* q, const double* k, const double* v,
                        const double* log_g, const double* beta,
                        const double* init_state, double scale,
                        const double* d_out, const double* d_final,
                        double* dq, double* dk_out, double* dv_out,
                        double* dlog_g, double* dbeta, double* d_init) {
  const int64_t n = u->n, h = u->h, len = u->len, sz = dk * dv;
  /* hist: len states; then S, P, dS, dP (dk x dv each), kv, delta, ddelta, dkv (dv), a (dk) */
  double* hist = (double*)malloc(sizeof(double) * ((len + 4) * sz + 4 * dv + dk));
  if (!hist) return -4;
  double* S = hist + len * sz;
  double* P = S + sz;
  double* dS = P + sz;
  double* dP = dS + sz;
  double* kv = dP + sz;
  double* delta = kv + dv;
  double* ddelta = delta + dv;
  double* dkv = ddelta + dv;
  double* a = dkv + dv;

  if (init_state)
    memcpy(S, init_state + (n * H + h) * sz, sizeof(double) * sz);
  else
    memset(S, 0, sizeof(double) * sz);

  /* forward, keeping the state before every token */
  for (int64_t s = 0; s < len; ++s) {
    const int64_t t = u->start + s;
    const double* kt = k + (t * H + h) * dk;
    const double* gt = log_g + (t * H + h) * dk;
    const double* vt = v + (t * H + h) * dv;
    const double bt = beta[t * H + h];
    memcpy(hist + s * sz, S, sizeof(double) * sz);
    for (int64_t i = 0; i < dk; ++i) {
      const double ai = exp(gt[i]);
      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] *= ai;
    }
    for (int64_t j = 0; j < dv; ++j) kv[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) kv[j] += S[i * dv + j] * kt[i];
    for (int64_t j = 0; j < dv; ++j) delta[j] = bt * (vt[j] - kv[j]);
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] += kt[i] * delta[j];
  }

  /* dL/dS after the last token */
  if (d_final)
    memcpy(dS, d_final + (n * H + h) * sz, sizeof(double) * sz);
  else
    memset(dS, 0, sizeof(double) * sz);

  for (int64_t s = len - 1; s >= 0; --s) {
    const int64_t t = u->start + s;
    const double* qt = q + (t * H + h) * dk;
    const double* kt = k + (t * H + h) * dk;
    const double* gt = log_g + (t * H + h) * dk;
    const double* vt = v + (t * H + h) * dv;
    const double bt = beta[t * H + h];
    const double* Sprev = hist + s * sz;
    double* dqt = dq + (t * H + h) * dk;
    double* dkt = dk_out + (t * H + h) * dk;
    double* dgt = dlog_g + (t * H + h) * dk;
    double* dvt = dv_out + (t * H + h) * dv;

    /* recompute this token's forward quantities from the state before it */
    for (int64_t i = 0; i < dk; ++i) {
      a[i] = exp(gt[i]);
      for (int64_t j = 0; j < dv; ++j) P[i * dv + j] = a[i] * Sprev[i * dv + j];
    }
    for (int64_t j = 0; j < dv; ++j) kv[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) kv[j] += P[i * dv + j] * kt[i];
    for (int64_t j = 0; j < dv; ++j) delta[j] = bt * (vt[j] - kv[j]);
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) S[i * dv + j] = P[i * dv + j] + kt[i] * delta[j];

    /* output o_t = scale S_t^T q_t */
    if (d_out) {
      const double* dot = d_out + (t * H + h) * dv;
      for (int64_t i = 0; i < dk; ++i) {
        double acc = 0.0;
        for (int64_t j = 0; j < dv; ++j) acc += S[i * dv + j] * dot[j];
        dqt[i] = scale * acc;
      }
      for (int64_t i = 0; i < dk; ++i)
        for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] += scale * qt[i] * dot[j];
    } else {
      for (int64_t i = 0; i < dk; ++i) dqt[i] = 0.0;
    }
    /* rank-1 update S_t = P + k_t delta^T */
    for (int64_t i = 0; i < dk; ++i) {
      double acc = 0.0;
      for (int64_t j = 0; j < dv; ++j) acc += dS[i * dv + j] * delta[j];
      dkt[i] = acc;
    }
    for (int64_t j = 0; j < dv; ++j) ddelta[j] = 0.0;
    for (int64_t i = 0; i < dk; ++i)
      for (int64_t j = 0; j < dv; ++j) ddelta[j] += dS[i * dv + j] * kt[i];
    /* scaled error delta = beta_t (v_t - kv) */
    {
      double acc = 0.0;
      for (int64_t j = 0; j < dv; ++j) acc += ddelta[j] * (vt[j] - kv[j]);
      dbeta[t * H + h] = acc;
    }
    for (int64_t j = 0; j < dv; ++j) {
      dvt[j] = bt * ddelta[j];
      dkv[j] = -bt * ddelta[j];
    }
    /* read-back kv = P^T k_t */
    for (int64_t i = 0; i < dk; ++i) {
      double acc = 0.0;
      for (int64_t j = 0; j < dv; ++j) {
        dP[i * dv + j] = dS[i * dv + j] + kt[i] * dkv[j];
        acc += P[i * dv + j] * dkv[j];
      }
      dkt[i] += acc;
    }
    /* decay P = Diag(exp(g_t)) S_{t-1} */
    for (int64_t i = 0; i < dk; ++i) {
      double acc = 0.0;
      for (int64_t j = 0; j < dv; ++j) acc += dP[i * dv + j] * Sprev[i * dv + j];
      dgt[i] = a[i] * acc;
      for (int64_t j = 0; j < dv; ++j) dS[i * dv + j] = a[i] * dP[i * dv + j];
    }
  }
  if (d_init) memcpy(d_init + (n * H + h) * sz, dS, sizeof(double) * sz);
  free(hist);
  return 0;
}

int kda_oracle_backward(int64_t num_seqs, int64_t seq_len, int64_t num_heads,
                        int64_t dk, int64_t dv, const double* q, const double* k,
                        const double* v, const double* log_g, const double* beta,
                        const double* init_state, const int64_t* cu_seqlens,
                        double scale, const double* d_out, const double* d_final,
                        double* dq, double* dk_out, double* dv_out,
                        double* dlog_g, double* dbeta, double* d_init,
                        int n_threads) {
  if (!q || !k || !v || !log_g || !beta || !dq || !dk_out || !dv_out || !dlog_g || !dbeta)
    return -1;
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
  for (int64_t n = 0; n < num_seqs; ++n)
    for (int64_t h = 0; h < num_heads; ++h) {
      unit_t* u = &units[n * num_heads + h];
      u->n = n;
      u->h = h;
      u->start = cu_seqlens ? cu_seqlens[n] : n * seq_len;
      u->len = cu_seqlens ? cu_seqlens[n + 1] - cu_seqlens[n] : seq_len;
    }
  qsort(units, (size_t)n_units, sizeof(unit_t), by_len_desc);

  int failed = 0;
#ifdef _OPENMP
  const int nt = kda_oracle_threads(n_threads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 1)
#endif
  for (int64_t u = 0; u < n_units; ++u) {
    if (run_unit_bwd(&units[u], num_heads, dk, dv, q, k, v, log_g, beta, init_state, scale,
                     d_out, d_final, dq, dk_out, dv_out, dlog_g, dbeta, d_init) != 0) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
    }
  }
  free(units);
  return failed ? -4 : 0;
}

/* The short causal depthwise convolution, one (document, channel) at a time:
 * the extended sequence (cache, then the document's inputs) is walked token by
 * token and each output is the K-tap dot product ending at that token. */
int kda_oracle_short_conv(int64_t num_seqs, int64_t seq_len, int64_t channels,
                          int64_t K, const double* x, const double* w,
                          const int64_t* cu_seqlens, const double* init_cache,
                          int act, double* y, double* final_cache, int n_threads) {
  if (!x || !w || !y) return -1;
  if (num_seqs < 0 || seq_len < 0 || channels <= 0 || K < 1 || (act != 0 && act != 1)) return -2;
  if (cu_seqlens) {
    if (cu_seqlens[0] != 0 || cu_seqlens[num_seqs] != seq_len) return -3;
    for (int64_t n = 0; n < num_seqs; ++n)
      if (cu_seqlens[n + 1] < cu_seqlens[n]) return -3;
  }
  const int64_t M = K - 1; /* cached inputs per (document, channel) */
  int failed = 0;
#ifdef _OPENMP
  const int nt = kda_oracle_threads(n_threads);
#pragma omp parallel for num_threads(nt) schedule(dynamic, 16)
#endif
  for (int64_t nc = 0; nc < num_seqs * channels; ++nc) {
    const int64_t n = nc / channels, c = nc % channels;
    const int64_t start = cu_seqlens ? cu_seqlens[n] : n * seq_len;
    const int64_t len = cu_seqlens ? cu_seqlens[n + 1] - cu_seqlens[n] : seq_len;
    /* extended sequence: M cached inputs, then the document's len inputs */
    double* xe = (double*)malloc(sizeof(double) * (size_t)(M + len + 1));
    if (!xe) {
#ifdef _OPENMP
#pragma omp atomic write
#endif
      failed = 1;
      continue;
    }
    for (int64_t m = 0; m < M; ++m)
      xe[m] = init_cache ? init_cache[(n * channels + c) * M + m] : 0.0;
    for (int64_t t = 0; t < len; ++t) xe[M + t] = x[(start + t) * channels + c];
    for (int64_t t = 0; t < len; ++t) {
      /* window xe[t .. t + M] (in extended indices) ends at the document's token t */
      double acc = 0.0;
      for (int64_t j = 0; j < K; ++j) acc += w[c * K + j] * xe[t + j];
      if (act == 1) acc = acc / (1.0 + exp(-acc));
      y[(start + t) * channels + c] = acc;
    }
    if (final_cache)
      for (int64_t m = 0; m < M; ++m) final_cache[(n * channels + c) * M + m] = xe[len + m];
    free(xe);
  }
  return failed ? -4 : 0;
}

/* Gated per-head RMSNorm, one row at a time: the mean square over the head
 * dim, the normalised row times the weight, then the sigmoid gate. */
int kda_oracle_gated_rmsnorm(int64_t rows, int64_t D, const double* o, const double* g,
                             const double* w, double eps, double* y) {
  if (!o || !g || !w || !y) return -1;
  if (rows < 0 || D <= 0 || !(eps >= 0.0)) return -2;
  for (int64_t r = 0; r < rows; ++r) {
    const double* orow = o + r * D;
    double ms = 0.0;
    for (int64_t i = 0; i < D; ++i) ms += orow[i] * orow[i];
    ms /= (double)D;
    const double inv = 1.0 / sqrt(ms + eps);
    for (int64_t i = 0; i < D; ++i) {
      const double gate = 1.0 / (1.0 + exp(-g[r * D + i]));
      y[r * D + i] = orow[i] * inv * w[i] * gate;
    }
  }
  return 0;
}

/* One row divided by its L2 norm, eps inside the root. */
static void l2norm_row(int64_t D, double eps, const double* x, double* y) {
  double ss = 0.0;
  for (int64_t i = 0; i < D; ++i) ss += x[i] * x[i];
  const double inv = 1.0 / sqrt(ss + eps);
  for (int64_t i = 0; i < D; ++i) y[i] = x[i] * inv;
}

int kda_oracle_qk_l2norm(int64_t rows, int64_t D, double eps, const double* q, const double* k,
                         double* qn, double* kn) {
  if (!q || !k || !qn || !kn) return -1;
  if (rows < 0 || D <= 0 || !(eps >= 0.0)) return -2;
  for (int64_t r = 0; r < rows; ++r) {
    l2norm_row(D, eps, q + r * D, qn + r * D);
    l2norm_row(D, eps, k + r * D, kn + r * D);
  }
  return 0;
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
