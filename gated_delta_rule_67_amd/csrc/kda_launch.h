// kda_launch.h -- host-side launchers of the libkda kernels (internal, C++).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

// Arguments of one decode / verify launch; shapes already validated.
struct StepLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* log_g;
  const float* beta;
  float* state;
  void* out;
  int num_seqs;
  int n_tok;
  int num_heads;
  int d;        // dk == dv
  bool bf16;    // q/k/v element type
  float scale;
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
  int32_t* doc_order;         // workspace: longest-first document order (packed only)
  int num_seqs;               // dense B or packed N
  int seq_len;                // dense T or packed total
  int num_heads;
  int d;
  bool bf16;
  float scale;
};

hipError_t launch_step(const StepLaunch& a, hipStream_t stream);
// Prefill through the token-recurrent kernel (any dtype / d).
hipError_t launch_chunk_recurrent(const ChunkLaunch& a, hipStream_t stream);
// Prefill through the chunked MFMA kernel (bf16 q/k/v, d = 128).
hipError_t launch_chunk_mfma(const ChunkLaunch& a, hipStream_t stream);
// Whether the chunked MFMA kernel takes this problem.
bool chunk_mfma_supported(const ChunkLaunch& a);

// Workspace bytes of the chunked prefill for a packed problem with n_docs documents.
size_t chunk_workspace_bytes(int n_docs, bool packed);

}  // namespace kda
