// kda_chunk.hip -- chunked (64-token) prefill of the KDA recurrence on MFMA (gfx950).
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {

size_t chunk_workspace_bytes(int n_docs, bool packed) {
  if (!packed || n_docs <= 0) return 0;
  return ((static_cast<size_t>(n_docs) * sizeof(int32_t) + 255) / 256) * 256;
}

bool chunk_mfma_supported(const ChunkLaunch&) { return false; }

hipError_t launch_chunk_mfma(const ChunkLaunch&, hipStream_t) { return hipErrorNotSupported; }

}  // namespace kda
