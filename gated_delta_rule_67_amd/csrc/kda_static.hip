// kda_static.hip -- kda_chunk_fwd_static: the chunked prefill with its scratch
// in a fixed device array instead of a caller workspace, for callers that
// cannot allocate (code under HIP graph capture, tight serving loops).
//
// The array is a file-scope __device__ symbol.  Host code never passes its
// name to a kernel (in host code the name is only a host-side stand-in): the
// array's device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and that address is what
// the kernels receive.  Every call on a device shares its array; calls that
// overlap on one device (other streams, other threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_launch.h"

namespace {

constexpr int MAX_DEV = 64;

__device__ __align__(256) unsigned char scratch[KDA_STATIC_SCRATCH_BYTES];

std::mutex g_lock;
void* g_scratch[MAX_DEV] = {};  // device address of `scratch` per device, once looked up

// The current device's address of `scratch` (looked up on first use).
hipError_t scratch_of_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

extern "C" kda_status kda_chunk_fwd_static(const kda_desc* desc, const void* q, const void* k, const void* v,
                                           const float* log_g, const float* beta, const float* init_state,
                                           const int32_t* cu_seqlens, void* out, float* final_state, void* stream) {
  void* ws = nullptr;
  const hipError_t e = scratch_of_current_device(&ws);
  if (e != hipSuccess) return kda::fail_hip("kda_chunk_fwd_static", "looking up the fixed scratch", e);
  return kda::chunk_fwd_checked(desc, q, k, v, log_g, beta, init_state, cu_seqlens, out, final_state, stream, ws,
                                KDA_STATIC_SCRATCH_BYTES, true, "kda_chunk_fwd_static");
}
