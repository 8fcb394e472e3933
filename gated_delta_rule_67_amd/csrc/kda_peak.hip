// kda_peak.hip -- on-box peak probe for the benchmark's rooflines.
//
// Not part of libkda: built into its own libkda_peak.so, loaded only by the
// benchmark, which times it to report the dense 16-bit MFMA rate this GPU
// actually sustains next to the published 2.5 PFLOP/s.  Each wave issues
// `iters` rounds of eight independent v_mfma_f32_16x16x32_f16 (16384 FLOP
// each; eight accumulators hide the instruction's latency), with nothing but
// loop control beside them.
#include <hip/hip_runtime.h>

namespace {

typedef _Float16 f16;
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;  // four waves per workgroup

__global__ void __launch_bounds__(NT) mfma_loop_kernel(int iters, float* sink) {
  f16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = static_cast<f16>(1e-3f * static_cast<float>((threadIdx.x + e) & 7));
    b[e] = static_cast<f16>(1e-3f * static_cast<float>(e));
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  // data-dependent store: the loop cannot be removed, and in practice never writes
  if (s == 1234567.0f) sink[blockIdx.x * NT + threadIdx.x] = s;
}

}  // namespace

extern "C" {

// FLOP of one launch: blocks * 4 waves * iters * 8 * 16384.  sink: device
// buffer of blocks * 256 floats.  Returns the hipError_t of the launch.
int kda_peak_mfma_f16(int blocks, int iters, float* sink, void* stream) {
  if (blocks <= 0 || iters <= 0 || !sink) return static_cast<int>(hipErrorInvalidValue);
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(static_cast<unsigned>(blocks)), dim3(NT), 0,
                     static_cast<hipStream_t>(stream), iters, sink);
  return static_cast<int>(hipGetLastError());
}

}  // extern "C"
