// kda_launch.h -- host-side launchers of the libkda kernels (internal, C++).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kda.h"

namespace kda {

// The gated RMSNorm applied to a prefill's output (kda_chunk_fwd_gated_norm).
struct OutNorm {
  const void* gate;      // like out, element type qkv_dtype
  const float* weight;   // [dv]
  float eps;
};

// kda_chunk_fwd's validation and launch with the workspace given explicitly:
// the caller's (desc->workspace) or the library's fixed scratch (fixed_ws,
// ws_bytes = its capacity).  norm (or null): the output is normalised in
// place by the gated RMSNorm after the prefill.  fn names the entry point in
// error messages.
kda_status chunk_fwd_checked(const kda_desc* d, const void* q, const void* k, const void* v, const float* log_g,
                             const float* beta, const float* init_state, const int32_t* cu_seqlens, void* out,
                             float* final_state, void* stream, void* ws, size_t ws_bytes, bool fixed_ws,
                             const char* fn, const OutNorm* norm = nullptr);
// Records "fn: what: <HIP error>" as the thread's last error; returns KDA_ERR_HIP.
kda_status fail_hip(const char* fn, const char* what, hipError_t e);

// Arguments of one decode / verify launch; shapes already validated.
struct StepLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const float* beta;
  float* state;        // read, and written back unless keep_state
  void* out;
  float* deltas;       // per-row delta [N, n_tok, H, dv], or null
  bool keep_state;     // true: the state is only read (speculative rows)
  int num_seqs;
  int n_tok;
  int num_heads;
  int d;        // dk == dv
  bool bf16;    // q/k/v element type
  bool out_bf16;  // out element type (else fp32)
  bool l2;      // L2-normalise the q and k rows first
  float scale;
};

// Arguments of one commit of accepted rows; shapes already validated.
struct CommitLaunch {
  const void* k;
  const float* log_g;
  const float* deltas;
  const int32_t* accept;  // device [N]
  float* state;
  int num_seqs;
  int n_tok;
  int num_heads;
  int d;
  bool bf16;
  bool l2;      // L2-normalise the k rows first
};

// Arguments of one chunked prefill launch; shapes already validated.
struct ChunkLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const float* beta;
  const float* init_state;    // may be null (zeros)
  const int32_t* cu_seqlens;  // may be null (dense)
  void* out;
  float* final_state;         // may be null
  void* workspace;            // caller scratch (already checked to be large enough)
  int num_seqs;               // dense B or packed N
  int seq_len;                // dense T or packed total
  int num_heads;
  int d;
  bool bf16;
  bool out_bf16;              // out element type (else fp32)
  bool l2;                    // L2-normalise the q and k rows first
  float scale;
};

hipError_t launch_step(const StepLaunch& a, hipStream_t stream);
hipError_t launch_commit(const CommitLaunch& a, hipStream_t stream);
// Prefill through the token-recurrent kernel (any dtype / d).  No workspace.
hipError_t launch_chunk_recurrent(const ChunkLaunch& a, hipStream_t stream);

// Prefill in two passes: per-chunk preparation over all chunks at once, then
// the serial state scan (bf16 q/k/v, d = 128).
hipError_t launch_chunk_twopass(const ChunkLaunch& a, hipStream_t stream);
bool twopass_supported(const ChunkLaunch& a);
size_t twopass_workspace_bytes(int num_seqs, int seq_len, int num_heads, bool packed);

// Arguments of one reverse-mode launch of the chunked prefill; shapes
// already validated.  Gradients are fp32 and laid out like their inputs.
struct BwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const float* beta;
  const float* init_state;    // may be null (zeros)
  const int32_t* cu_seqlens;  // may be null (dense)
  const float* d_out;
  const float* d_final;       // may be null (zeros)
  float* dq;
  float* dk;
  float* dv;
  float* dlog_g;
  float* dbeta;
  float* d_init;              // may be null (not written)
  void* workspace;            // caller scratch (already checked to be large enough)
  int num_seqs;
  int seq_len;
  int num_heads;
  int d;
  bool bf16;
  float scale;
};

hipError_t launch_chunk_bwd(const BwdLaunch& a, hipStream_t stream);
bool bwd_supported(const BwdLaunch& a);
size_t bwd_workspace_bytes(int num_seqs, int seq_len, int num_heads, int d, bool packed);

// Arguments of one short causal depthwise convolution; shapes already validated.
struct ConvLaunch {
  const void* x;
  const float* weight;        // [channels, kernel_size]
  const int32_t* cu_seqlens;  // may be null (dense)
  const float* init_cache;    // may be null (zeros)
  float* final_cache;         // may be null
  void* out;
  int num_seqs;
  int seq_len;
  int channels;
  int kernel_size;            // 1..8
  int activation;             // 0 identity, 1 SiLU
  bool bf16;                  // x and out element type
};

hipError_t launch_short_conv(const ConvLaunch& a, hipStream_t stream);

// Arguments of one gated per-head RMSNorm; shapes already validated.
struct NormLaunch {
  const void* o;        // [rows, d], fp32, or bf16 when o_bf16; may be out
  const void* gate;     // [rows, d]
  const float* weight;  // [d]
  void* out;            // [rows, d]
  int64_t rows;
  int d;
  float eps;
  bool gate_bf16;
  bool out_bf16;
  bool o_bf16;
};

hipError_t launch_gated_rmsnorm(const NormLaunch& a, hipStream_t stream);


}  // namespace kda
