/*
 * kda.h -- C ABI of libkda, the MI355X (gfx950) Kimi Delta Attention mixer.
 *
 * The operation (GLM-5.3-Flash model notes, Glm5NextTextLinearAttention snippet;
 * NeMo glm5_next.layers, `_torch_recurrent_kda`): for every unit u = (sequence or
 * packed document n, head h) a per-head fp32 state S[dk][dv] (row i = key
 * channel i, column j = value channel j) runs, token by token,
 *
 *     S[i,:]   *= exp(log_g[t,h,i])              each key channel decays by its gate
 *     kv        = S^T k_t                        the state's prediction for k_t
 *     delta     = beta[t,h] * (v_t - kv)         scaled prediction error
 *     S        += k_t delta^T                    rank-1 delta-rule update
 *     out[t,h,:] = scale * S^T q_t               read from the updated state
 *
 * Packed documents never share state: each starts from its own initial state
 * (NeMo glm5_next.layers, `Glm5NextLinearAttention.forward`: KDA runs "without
 * crossing documents"; `_torch_recurrent_kda`: packed boundaries reset the state).
 *
 * Conventions for every entry point
 *  - Tensors are row-major with the last axis contiguous:
 *      q, k, log_g : [batch, seq, heads, dk]     v, out : [batch, seq, heads, dv]
 *      beta        : [batch, seq, heads]         states : [N, heads, dk, dv]
 *    (the [batch, sequence, heads, head_dim] layout of `_torch_recurrent_kda`).
 *  - q, k, v have element type desc->qkv_dtype (fp32 or bf16); log_g, beta and
 *    states are fp32; out has element type desc->out_dtype: fp32, or bf16
 *    (the fp32 result rounded once to nearest even) for kda_chunk_fwd,
 *    kda_step and kda_step_rows.
 *  - Every data pointer is a DEVICE pointer owned by the caller and must be
 *    16-byte aligned.  The library never allocates, frees or caches device
 *    memory; scratch comes from desc->workspace.  The descriptor itself is host
 *    memory and is read only during the call.
 *  - All work is enqueued on `stream` (a hipStream_t; NULL = the null stream).
 *    KDA_OK means "validated and enqueued"; faults inside a kernel surface at
 *    the caller's next synchronisation.  No entry point synchronises.
 *  - Host-visible arguments are validated before anything is enqueued; a
 *    non-OK status leaves every output untouched.  kda_last_error() then
 *    describes the failure (thread-local string).  Nothing throws or aborts
 *    across the ABI.
 *  - Preconditions the library does not check (they live in device memory):
 *    log_g <= 0 (log_g = -inf allowed), cu_seqlens well formed.
 *  - Supported: dk == dv in {16, 32, 64, 128}; qkv_dtype fp32 or bf16;
 *    out_dtype as above.  Anything else returns KDA_ERR_UNSUPPORTED.
 *  - desc->flags selects options (KDA_FLAG_*); unknown bits return
 *    KDA_ERR_UNSUPPORTED.
 *  - Environment: KDA_VALIDATE=1 makes kda_chunk_fwd and kda_step check their
 *    device-resident preconditions and results (see below); it synchronises
 *    the stream and is meant for debugging only.
 */
#ifndef KDA_H
#define KDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_ABI_VERSION 7

/* desc->flags bits.
 * KDA_FLAG_QK_L2NORM: every (token, head) row of q and of k is divided by
 *   sqrt(sum of its squares + 1e-6) inside the kernels before the recurrence
 *   uses it (the optional normalisation step in front of the mixer; the pages
 *   do not print it, and this plain L2 form with eps inside the root is the
 *   reading taken).  Honoured by kda_chunk_fwd, kda_step, kda_step_rows and
 *   kda_step_commit (which normalises the k rows it replays); kda_chunk_bwd
 *   returns KDA_ERR_UNSUPPORTED with it. */
#define KDA_FLAG_QK_L2NORM 1u
#define KDA_QK_L2NORM_EPS 1e-6f

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = 1,        /* a required pointer is NULL                      */
  KDA_ERR_SHAPE = 2,       /* a dimension is <= 0, too large, or inconsistent */
  KDA_ERR_DTYPE = 3,       /* unknown dtype code                              */
  KDA_ERR_ALIGN = 4,       /* a data pointer is not 16-byte aligned           */
  KDA_ERR_WORKSPACE = 5,   /* workspace missing or smaller than required      */
  KDA_ERR_UNSUPPORTED = 6, /* valid but not implemented (dk != dv, d, out)    */
  KDA_ERR_HIP = 7          /* a HIP runtime call or kernel launch failed      */
} kda_status;

typedef enum { KDA_F32 = 0, KDA_BF16 = 1 } kda_dtype;

/* Problem descriptor (host memory). */
typedef struct kda_desc {
  int32_t num_seqs;  /* dense: batch B; packed: number of documents N           */
  int32_t seq_len;   /* dense: tokens per sequence T; packed: total tokens.
                        Not read by kda_step (it takes n_tok)                   */
  int32_t num_heads; /* H, shared by q, k, v                                     */
  int32_t dk;        /* key / query head dim  (rows of S)                        */
  int32_t dv;        /* value head dim        (columns of S)                     */
  int32_t qkv_dtype; /* kda_dtype of q, k, v                                     */
  int32_t out_dtype; /* kda_dtype of out                                        */
  float scale;       /* output scale; 0 selects dk^-0.5                          */
  void* workspace;   /* device scratch of kda_chunk_fwd, at least
                        kda_chunk_workspace_bytes(desc, packed) bytes          */
  size_t workspace_bytes;
  uint32_t flags;    /* KDA_FLAG_* bits; 0 = none                                */
  uint32_t reserved; /* must be 0                                                */
} kda_desc;

/* ABI version of the loaded library (KDA_ABI_VERSION it was built with). */
int kda_abi_version(void);

/* Static description of a status code. Never NULL. */
const char* kda_status_string(kda_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* kda_last_error(void);

/* Device scratch bytes kda_chunk_fwd needs for this descriptor; packed != 0
 * for a call with cu_seqlens (desc->seq_len = total tokens, num_seqs =
 * documents), 0 for a dense batch.  The descriptor alone cannot tell the two
 * apart (num_seqs and seq_len mean different things in each), and the slot
 * count differs: dense B * ceil(T/64), packed ceil(T/64) + N.  For bf16 q/k/v with d = 128 the chunked
 * prefill stages fp16 per-chunk operands there: 73 KiB per 64-token
 * chunk and head (dense: B * ceil(T/64) chunks; packed: ceil(T/64) + N, an
 * upper bound), plus a few bytes per document when packed.  Other
 * configurations need at most a few bytes per document (0 for a dense
 * batch; desc->workspace may then be NULL).  The figure is for the
 * evaluation path in force when it is queried (see KDA_PREFILL_PATH below).
 * The workspace is scratch: its contents on entry do not matter and are
 * clobbered.  Returns 0 for a NULL or invalid descriptor. */
size_t kda_chunk_workspace_bytes(const kda_desc* desc, int packed);

/*
 * Chunked prefill (dense batch or packed varlen).
 *
 *   q, k, log_g  [B, T, H, dk];  v [B, T, H, dv];  beta [B, T, H]
 *   init_state   [N, H, dk, dv] fp32, or NULL for zeros
 *   cu_seqlens   device int32 [N+1] (cu[0] = 0, non-decreasing, cu[N] = T), or
 *                NULL for a dense batch of B = num_seqs sequences of T tokens
 *                (packed: B = 1, T = seq_len total tokens, N = num_seqs docs)
 *   out          [B, T, H, dv] (out_dtype)
 *   final_state  [N, H, dk, dv] fp32, or NULL to skip; may alias init_state
 *                (in-place resume) but nothing else
 *
 * Evaluated in chunks of 64 tokens (within a document) with fp32 state and fp32
 * accumulation; out must not alias any input.  Zero-length documents are
 * allowed (their final state is their initial state).
 *
 * Evaluation path: bf16 q/k/v with d = 128 take the two-pass chunked kernels
 * (per-chunk operands staged in the workspace); other inputs take the
 * token-recurrent kernel.  The chunked path's serial pass runs four 32-column
 * workgroups per (sequence or document, head): eight-wave ones, or four-wave
 * ones two to a CU when there are more such tiles than 256.  The environment
 * variable KDA_PREFILL_PATH, read at every call, is a test and diagnosis
 * switch: "recurrent" forces the token-recurrent kernel, "tile8" or "tile4" a
 * form of the serial pass.  A workspace smaller than the selected path needs
 * returns KDA_ERR_WORKSPACE before anything is enqueued.
 *
 * KDA_VALIDATE=1 (read at every call): before the launch, the call copies
 * cu_seqlens and log_g to the host and returns KDA_ERR_SHAPE if cu_seqlens
 * is not [0, ..., seq_len] non-decreasing or any log_g is NaN or positive;
 * it fills out and final_state with NaN first, and after the kernels (a
 * stream synchronisation) returns KDA_ERR_HIP if any element of out or
 * final_state was left unwritten or is not finite.
 */
kda_status kda_chunk_fwd(const kda_desc* desc, const void* q, const void* k,
                         const void* v, const float* log_g, const float* beta,
                         const float* init_state, const int32_t* cu_seqlens,
                         void* out, float* final_state, void* stream);

/*
 * kda_chunk_fwd with the gated per-head RMSNorm applied to its output in the
 * same call (NeMo glm5_next.layers: the mixer output passes
 * `_TorchRMSNormGated` before the output projection; kda_gated_rmsnorm below
 * is the same norm as a call of its own).  out receives, per token t and
 * head h, with o[t,h,:] what kda_chunk_fwd would write:
 *
 *     out[t,h,i] = o[t,h,i] / sqrt(mean(o[t,h,:]^2) + eps) * norm_weight[i] * sigmoid(gate[t,h,i])
 *
 *   gate         [B, T, H, dv], element type desc->qkv_dtype
 *   norm_weight  [dv] fp32 (shared by the heads);  eps >= 0
 *   out          [B, T, H, dv], out_dtype
 * o is first stored into out in out_dtype and then normalised there in place
 * by a second pass on the same stream (with bf16 out: o rounded once to bf16,
 * the normalised value rounded once more).  Every kda_chunk_fwd configuration
 * is supported.  Everything else (arguments, workspace, final_state, errors,
 * KDA_VALIDATE on the prefill) is as for kda_chunk_fwd.  out must not alias
 * gate or norm_weight.
 */
kda_status kda_chunk_fwd_gated_norm(const kda_desc* desc, const void* q, const void* k,
                                    const void* v, const float* log_g, const float* beta,
                                    const float* init_state, const int32_t* cu_seqlens,
                                    const void* gate, const float* norm_weight, float eps,
                                    void* out, float* final_state, void* stream);

/*
 * kda_chunk_fwd without a workspace, for callers that cannot allocate (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, results and errors as kda_chunk_fwd, except
 * that desc->workspace and desc->workspace_bytes are ignored: the scratch is
 * a fixed array of KDA_STATIC_SCRATCH_BYTES inside the library, one per
 * device, held until the process ends.  A problem needing more scratch than
 * that (kda_chunk_workspace_bytes) returns KDA_ERR_WORKSPACE before
 * anything is enqueued.  Calls allocate nothing (no hipMalloc, no hipFree).
 * Every call on a device shares that device's array: calls that may overlap
 * on one device (different streams, different host threads) race on it and
 * must be ordered by the caller.  The array's contents on entry do not
 * matter (every byte a call reads it wrote first).
 */
#define KDA_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
kda_status kda_chunk_fwd_static(const kda_desc* desc, const void* q, const void* k,
                                const void* v, const float* log_g, const float* beta,
                                const float* init_state, const int32_t* cu_seqlens,
                                void* out, float* final_state, void* stream);

/*
 * Decode / multi-row verify, updating the state in place.
 *
 *   q, k, log_g [N, n_tok, H, dk];  v [N, n_tok, H, dv];  beta [N, n_tok, H]
 *   state_inout [N, H, dk, dv] fp32, read once and written once
 *   out         [N, n_tok, H, dv] (out_dtype): row t's output, read from the
 *               state after rows 0..t of that sequence
 *
 * Rows of one sequence are applied in order t = 0 .. n_tok-1 (metrale
 * glm5next_layer invariants: verify row t uses slot t; decode is n_tok = 1).
 * N = desc->num_seqs; desc->seq_len is ignored; no workspace is used.
 * KDA_VALIDATE=1 checks log_g on the host first and the finiteness of out
 * and of the updated state after the kernel, as for kda_chunk_fwd.
 */
kda_status kda_step(const kda_desc* desc, const void* q, const void* k,
                    const void* v, const float* log_g, const float* beta,
                    float* state_inout, int32_t n_tok, void* out, void* stream);

/*
 * Speculative verify in two calls: score n_tok draft rows per sequence, then
 * keep only each sequence's accepted prefix (verify row t uses slot t:
 * metrale glm5next_layer invariants; rows past the accepted prefix must
 * leave no trace in the state).
 *
 * kda_step_rows: the outputs of rows 0 .. n_tok-1, exactly as kda_step would
 * produce them, WITHOUT changing the state; each row's
 * delta_t = beta_t (v_t - kv_t) is written so any prefix can be committed.
 *   q, k, log_g [N, n_tok, H, dk];  v [N, n_tok, H, dv];  beta [N, n_tok, H]
 *   state       [N, H, dk, dv] fp32, read only
 *   out         [N, n_tok, H, dv] (out_dtype)
 *   deltas      [N, n_tok, H, dv] fp32
 *
 * kda_step_commit: advance sequence n's state by its first accept[n] rows,
 * S <- Diag(exp(log_g_t)) S + k_t delta_t^T for t = 0 .. accept[n]-1 (the
 * state update of kda_step with the read-back already done), from the same
 * state kda_step_rows read.  With accept[n] = n_tok the result is kda_step's
 * final state; with accept[n] = 0 the state is left as it was.
 *   k, log_g    [N, n_tok, H, dk]: the rows given to kda_step_rows
 *   deltas      [N, n_tok, H, dv]: its output
 *   accept      device int32 [N]; values outside [0, n_tok] are clamped
 *   state_inout [N, H, dk, dv] fp32, updated in place
 * Neither call uses a workspace; out and deltas must not alias any input.
 */
kda_status kda_step_rows(const kda_desc* desc, const void* q, const void* k,
                         const void* v, const float* log_g, const float* beta,
                         const float* state, int32_t n_tok, void* out,
                         float* deltas, void* stream);

kda_status kda_step_commit(const kda_desc* desc, const void* k,
                           const float* log_g, const float* deltas,
                           const int32_t* accept, float* state_inout,
                           int32_t n_tok, void* stream);

/*
 * Reverse mode of kda_chunk_fwd (training): gradients of the scalar loss
 *
 *     L = sum(d_out * out) + sum(d_final_state * final_state)
 *
 * with respect to q, k, v, log_g, beta and init_state, for the same problem
 * (NeMo glm5_next.layers: `_torch_recurrent_kda` is documented as the
 * differentiable reference of this recurrence, and the layer is trained with
 * FSDP).  Inputs are exactly those of kda_chunk_fwd (same shapes, dtypes,
 * dense or packed, init_state NULL = zeros), plus
 *
 *   d_out          [B, T, H, dv] fp32, required when there are tokens
 *   d_final_state  [N, H, dk, dv] fp32, or NULL (the final state does not
 *                  enter the loss)
 *
 * Outputs, all fp32 whatever qkv_dtype is, laid out like their inputs:
 *   dq, dk, dlog_g [B, T, H, dk];  dv [B, T, H, dv];  dbeta [B, T, H]
 *   d_init_state   [N, H, dk, dv], or NULL to skip (zero-length documents
 *                  pass d_final_state through unchanged)
 * No output may alias an input or another output.  Everything is computed
 * in fp32 (fp32 matrix-core products, fp32 state); the forward is recomputed
 * inside the call, so out and final_state are not inputs.  desc->out_dtype
 * is ignored; desc->flags must be 0 (KDA_FLAG_QK_L2NORM: unsupported).
 *
 * desc->workspace must hold kda_chunk_bwd_workspace_bytes(desc, packed)
 * bytes whenever there are tokens or the problem is packed: about 465 KiB
 * per 64-token chunk and head at d = 128 (chunk entry states and their
 * gradients, per-chunk operands).  Its contents on entry do not matter.
 * Same status codes and preconditions as kda_chunk_fwd.
 */
size_t kda_chunk_bwd_workspace_bytes(const kda_desc* desc, int packed);
kda_status kda_chunk_bwd(const kda_desc* desc, const void* q, const void* k,
                         const void* v, const float* log_g, const float* beta,
                         const float* init_state, const int32_t* cu_seqlens,
                         const float* d_out, const float* d_final_state,
                         float* dq, float* dk, float* dv, float* dlog_g,
                         float* dbeta, float* d_init_state, void* stream);

/*
 * Short causal depthwise convolution that feeds q, k and v (NeMo
 * glm5_next.layers, `_TorchShortConvolution`: a depthwise causal Conv1d over
 * [batch, sequence, channels] that resets at packed boundaries; its width is
 * the config's linear_conv_kernel_dim).  For every sequence or document n,
 * channel c and token t of n (counted from the document start):
 *
 *     out[t, c] = act( sum_{j < K} weight[c, j] * xe[t - (K-1) + j, c] )
 *
 * where xe is the document's inputs preceded by its K-1 cached inputs
 * init_cache[n, c, 0..K-2] (oldest first; zeros when init_cache is NULL): the
 * window never reaches into another document.  Accumulation is fp32; out has
 * the element type of x.
 *
 *   desc         num_seqs (dense B / packed N), seq_len (dense T / packed total
 *                tokens) and qkv_dtype (element type of x and out) are read;
 *                the other fields are ignored
 *   channels     multiple of 8;  kernel_size K in [1, 8]
 *   activation   0 identity (the convolution as the pages name it), 1 SiLU
 *                applied to the sum (y / (1 + exp(-y)))
 *   x, out       [B, T, channels] (dense) or [1, T, channels] (packed);
 *                out must not alias x
 *   weight       [channels, K] fp32 (a depthwise Conv1d weight without its
 *                middle axis)
 *   cu_seqlens   device int32 [N+1] or NULL (dense), as for kda_chunk_fwd
 *   init_cache   [N, channels, K-1] fp32 or NULL
 *   final_cache  [N, channels, K-1] fp32 or NULL: the last K-1 entries of xe
 *                (the state a decode step continues from).  It may alias
 *                init_cache only for dense sequences of 1, 2, 4, 8, 16 or 32
 *                tokens (decode and verify); otherwise it must not.
 * No workspace.  Returns KDA_ERR_UNSUPPORTED for K outside [1, 8].
 */
kda_status kda_short_conv(const kda_desc* desc, int32_t channels, int32_t kernel_size,
                          int32_t activation, const void* x, const float* weight,
                          const int32_t* cu_seqlens, const float* init_cache, void* out,
                          float* final_cache, void* stream);

/*
 * Gated per-head RMSNorm on the mixer output (NeMo glm5_next.layers,
 * `_TorchRMSNormGated`: normalise [batch, sequence, heads, head_dim], then gate
 * with a sigmoid; the base RMSNorm accumulates the variance in fp32, and every
 * norm is x * w / rms, never x * (1 + w) / rms, per the metrale
 * glm5next_layer invariants).  For every token and head (a row of D = desc->dv
 * channels):
 *
 *     out[i] = o[i] / sqrt(mean(o^2) + eps) * weight[i] * sigmoid(gate[i])
 *
 *   desc    rows = num_seqs * seq_len * num_heads (a packed row: num_seqs = 1,
 *           seq_len = tokens); dv in {16, 32, 64, 128}; qkv_dtype is the
 *           element type of gate, out_dtype that of out (fp32 or bf16);
 *           dk, scale and the workspace are ignored
 *   o       [rows, D] fp32 (the output of kda_chunk_fwd or kda_step)
 *   gate    [rows, D];  weight [D] fp32 (shared by the heads);  eps >= 0
 *   out     [rows, D]; may be o itself when out_dtype is fp32, must not alias
 *           gate or weight
 * bf16 out is rounded to nearest even once, from the fp32 result.
 */
kda_status kda_gated_rmsnorm(const kda_desc* desc, const float* o, const void* gate,
                             const float* weight, float eps, void* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* KDA_H */
