// kda_norm.hip -- gated per-head RMSNorm on the mixer output (gfx950).
//
// NeMo glm5_next.layers, `_TorchRMSNormGated`: normalise [batch, sequence,
// heads, head_dim], then gate with a sigmoid.  Its base RMSNorm accumulates
// the variance in fp32, and every norm is x * w / rms (metrale glm5next_layer
// invariants), never x * (1 + w) / rms.  Per row (token, head) of D channels:
//
//     y[i] = o[i] / sqrt(mean(o^2) + eps) * w[i] * sigmoid(g[i])
//
// HBM-bound (o read, gate read, y written once).  A group of D / 8 lanes owns
// one row, 8 channels per lane; the sum of squares is reduced with shuffles
// inside the group.  o is fp32, or bf16 like out; out may be o itself (every
// element is read and written by the same lane).
#include "kda_common.h"
#include "kda_launch.h"
#include "kda_vec8.h"

namespace kda {
namespace {

constexpr int NTN = 256;

struct NormArgs {
  const void* o;
  const void* g;
  const float* w;
  void* out;
  int64_t rows;
  float eps;
};

template <int D, typename G, typename O, typename OIn>
__global__ void __launch_bounds__(NTN) gated_rmsnorm_kernel(NormArgs a) {
  constexpr int L = D / 8;  // lanes per row (divides 64)
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * NTN + threadIdx.x;
  const int64_t row = gid / L;
  const int part = static_cast<int>(gid - row * L);
  if (row >= a.rows) return;  // the lanes of one row leave together
  const int64_t off = row * D + 8 * part;
  float o[8], g[8], w[8];
  load8f(static_cast<const OIn*>(a.o) + off, o);
  load8f(static_cast<const G*>(a.g) + off, g);
  load8f(a.w + 8 * part, w);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += o[i] * o[i];
#pragma unroll
  for (int m = 1; m < L; m <<= 1) ss += __shfl_xor(ss, m, 64);
  const float inv = 1.f / sqrtf(ss * (1.f / D) + a.eps);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = o[i] * inv * w[i] / (1.f + exp_fast(-g[i]));
  store8f(static_cast<O*>(a.out) + off, y);
}

template <int D, typename OIn>
hipError_t launch_d(const NormLaunch& s, const NormArgs& a, hipStream_t stream) {
  const int64_t threads = a.rows * (D / 8);
  const unsigned blocks = static_cast<unsigned>((threads + NTN - 1) / NTN);
  if (s.gate_bf16) {
    if (s.out_bf16) hipLaunchKernelGGL((gated_rmsnorm_kernel<D, bf16_t, bf16_t, OIn>), dim3(blocks), dim3(NTN), 0, stream, a);
    else hipLaunchKernelGGL((gated_rmsnorm_kernel<D, bf16_t, float, OIn>), dim3(blocks), dim3(NTN), 0, stream, a);
  } else {
    if (s.out_bf16) hipLaunchKernelGGL((gated_rmsnorm_kernel<D, float, bf16_t, OIn>), dim3(blocks), dim3(NTN), 0, stream, a);
    else hipLaunchKernelGGL((gated_rmsnorm_kernel<D, float, float, OIn>), dim3(blocks), dim3(NTN), 0, stream, a);
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_o(const NormLaunch& s, const NormArgs& a, hipStream_t stream) {
  return s.o_bf16 ? launch_d<D, bf16_t>(s, a, stream) : launch_d<D, float>(s, a, stream);
}

}  // namespace

hipError_t launch_gated_rmsnorm(const NormLaunch& s, hipStream_t stream) {
  if (s.rows == 0) return hipSuccess;
  NormArgs a{s.o, s.gate, s.weight, s.out, s.rows, s.eps};
  switch (s.d) {
    case 16: return launch_o<16>(s, a, stream);
    case 32: return launch_o<32>(s, a, stream);
    case 64: return launch_o<64>(s, a, stream);
    case 128: return launch_o<128>(s, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
