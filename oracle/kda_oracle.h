/*
 * kda_oracle.h -- fp64 CPU oracle of the Kimi Delta Attention (KDA) recurrence.
 *
 * TEST INFRASTRUCTURE ONLY.  This library is the correctness reference that the
 * GPU path is checked against.  Only the test suite, the smoke entry point and
 * the benchmark's CPU-baseline leg may load or call it.  The product path
 * (libkda and its Python binding) never links, imports or calls it, and it
 * shares no code, header or table with the GPU path.
 *
 * What it computes (GLM-5.3-Flash model notes, the Glm5NextTextLinearAttention
 * snippet of the gated delta rule; NeMo glm5_next.layers, `_torch_recurrent_kda`):
 * for every unit u = (sequence or packed document n, head h), starting from
 * S = init_state[n,h] (or zeros), and for every token t of n in order
 *
 *     S[i,:]  *= exp(log_g[t,h,i])                 decay along the key axis
 *     kv[j]    = sum_i S[i,j] * k[t,h,i]           read back S^T k
 *     delta[j] = beta[t,h] * (v[t,h,j] - kv[j])    scaled prediction error
 *     S[i,j]  += k[t,h,i] * delta[j]               rank-1 delta-rule update
 *     out[t,h,j] = scale * sum_i S[i,j] * q[t,h,i] output from the updated state
 *
 * final_state[n,h] = S after the unit's last token.
 *
 * Layouts (row-major, last axis contiguous):
 *   q, k, log_g : [tokens, H, dk]      v, out : [tokens, H, dv]
 *   beta        : [tokens, H]          init_state, final_state : [N, H, dk, dv]
 * Dense mode (cu_seqlens == NULL): N sequences of seq_len tokens each, token
 * index n*seq_len + t.  Packed mode: cu_seqlens[N+1] (cu[0] = 0, non-decreasing,
 * cu[N] = total tokens) splits one packed row into N documents; the state is
 * reset to the document's own initial state at every document start.
 *
 * parity pins: every function here is pinned by the CPU tests (closed forms,
 * exact rational brute force, packed/split/linearity invariants; the backward
 * by central finite differences of the forward, a closed form and structural
 * invariants); none is "parity unpinned".
 */
#ifndef KDA_ORACLE_H
#define KDA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Returns 0 on success, a negative value on invalid arguments
 * (-1 NULL pointer, -2 bad dimension, -3 malformed cu_seqlens).
 * n_threads <= 0 uses the OpenMP default. */
int kda_oracle_forward(int64_t num_seqs, int64_t seq_len, int64_t num_heads,
                       int64_t dk, int64_t dv,
                       const double* q, const double* k, const double* v,
                       const double* log_g, const double* beta,
                       const double* init_state, const int64_t* cu_seqlens,
                       double scale, double* out, double* final_state,
                       int n_threads);

/* Reverse mode of kda_oracle_forward (NeMo glm5_next.layers: the reference
 * recurrence `_torch_recurrent_kda` is documented as differentiable, and the
 * KDA parameters are trained under FSDP).
 *
 * For the scalar loss L = sum(d_out * out) + sum(d_final * final_state),
 * returns dL/dq, dL/dk, dL/dv, dL/dlog_g, dL/dbeta and dL/dinit_state.  Same
 * shapes and layouts as the forward's inputs; d_out [tokens, H, dv] and
 * d_final [N, H, dk, dv] may be NULL (zeros); d_init may be NULL (not
 * written).  The forward is rerun per unit with the state before every token
 * kept (len * dk * dv doubles per unit in flight), then every token's step is
 * differentiated in reverse order.  Same return codes as the forward. */
int kda_oracle_backward(int64_t num_seqs, int64_t seq_len, int64_t num_heads,
                        int64_t dk, int64_t dv,
                        const double* q, const double* k, const double* v,
                        const double* log_g, const double* beta,
                        const double* init_state, const int64_t* cu_seqlens,
                        double scale, const double* d_out, const double* d_final,
                        double* dq, double* dk_out, double* dv_out,
                        double* dlog_g, double* dbeta, double* d_init,
                        int n_threads);

/* Short causal depthwise convolution that feeds q, k and v (NeMo
 * glm5_next.layers, `_TorchShortConvolution`: a depthwise causal Conv1d over
 * [batch, sequence, channels] that resets at packed boundaries; its width is
 * the config's linear_conv_kernel_dim).  For every sequence or document n,
 * channel c and token t of n (t counted from the document start),
 *
 *     y[t, c] = act( sum_{j=0}^{K-1} w[c, j] * xe[t - (K-1) + j, c] )
 *
 * where xe is the document's inputs preceded by its K-1 cached inputs
 * init_cache[n, c, 0..K-2] (oldest first; zeros when init_cache is NULL), so
 * the window never reaches into another document.  act = identity (0) or
 * SiLU, y / (1 + exp(-y)) (1).  final_cache[n, c, m] = xe[len - (K-1) + m, c]
 * (the last K-1 entries of the extended sequence), if not NULL.
 * Layouts: x, y [tokens, channels] (dense: token n*seq_len + t); w
 * [channels, K]; caches [N, channels, K-1].  Same return codes as the forward
 * (-2 also for K < 1 or an unknown act). */
int kda_oracle_short_conv(int64_t num_seqs, int64_t seq_len, int64_t channels,
                          int64_t K, const double* x, const double* w,
                          const int64_t* cu_seqlens, const double* init_cache,
                          int act, double* y, double* final_cache, int n_threads);

/* Gated per-head RMSNorm on the mixer output (NeMo glm5_next.layers,
 * `_TorchRMSNormGated`: normalise [batch, sequence, heads, head_dim], then
 * gate with a sigmoid; its base RMSNorm accumulates the variance in fp32, and
 * the metrale glm5next_layer invariants fix every norm as x * w / rms, never
 * x * (1 + w) / rms).  For every row r (a token and head) of head_dim D:
 *
 *     y[r, i] = o[r, i] / sqrt(mean_i(o[r, :]^2) + eps) * w[i] * sigmoid(g[r, i])
 *
 * o, g, y: [rows, D]; w: [D].  Returns 0, or -1 NULL pointer / -2 bad size. */
int kda_oracle_gated_rmsnorm(int64_t rows, int64_t D, const double* o, const double* g,
                             const double* w, double eps, double* y);

/* Number of OpenMP threads a call with n_threads would use. */
/* L2 normalisation of the query and key rows, the optional first step of the
 * mixer (the pages do not print it; the reading taken is the plain one: each
 * row of head_dim D, one token of one head, divided by its Euclidean norm
 * with eps inside the root):
 *
 *     qn[r, i] = q[r, i] / sqrt(sum_i q[r, :]^2 + eps),   kn likewise from k
 *
 * q, k, qn, kn: [rows, D].  The recurrence then runs on (qn, kn) unchanged.
 * Returns 0, or -1 NULL pointer / -2 bad size. */
int kda_oracle_qk_l2norm(int64_t rows, int64_t D, double eps, const double* q, const double* k,
                         double* qn, double* kn);

int kda_oracle_threads(int n_threads);

#ifdef __cplusplus
}
#endif
#endif /* KDA_ORACLE_H */
