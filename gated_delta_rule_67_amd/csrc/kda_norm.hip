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
// inside the group.
#include "kda_common.h"
#include "kda_launch.h"

namespace kda {
namespace {

constexpr int NTN = 256;

struct NormArgs {
  const float* o;
  const void* g;
  const float* w;
  void* out;
  int64_t rows;
  float eps;
};

__device__ __forceinline__ void ld8(const float* p, float (&v)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void ld8(const bf16_t* p, float (&v)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x); v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
  v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z); v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}
__device__ __forceinline__ void st8(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
// fp32 -> bf16, round to nearest even (finite inputs)
__device__ __forceinline__ uint32_t to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ void st8(bf16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = to_bf16_bits(v[0]) | (to_bf16_bits(v[1]) << 16);
  u.y = to_bf16_bits(v[2]) | (to_bf16_bits(v[3]) << 16);
  u.z = to_bf16_bits(v[4]) | (to_bf16_bits(v[5]) << 16);
  u.w = to_bf16_bits(v[6]) | (to_bf16_bits(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}

template <int D, typename G, typename O>
__global__ void __launch_bounds__(NTN) gated_rmsnorm_kernel(NormArgs a) {
  constexpr int L = D / 8;  // lanes per row (divides 64)
  const int64_t gid = static_cast<int64_t>(blockIdx.x) * NTN + threadIdx.x;
  const int64_t row = gid / L;
  const int part = static_cast<int>(gid - row * L);
  if (row >= a.rows) return;  // the lanes of one row leave together
  const int64_t off = row * D + 8 * part;
  float o[8], g[8], w[8];
  ld8(a.o + off, o);
  ld8(static_cast<const G*>(a.g) + off, g);
  ld8(a.w + 8 * part, w);
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) ss += o[i] * o[i];
#pragma unroll
  for (int m = 1; m < L; m <<= 1) ss += __shfl_xor(ss, m, 64);
  const float inv = 1.f / sqrtf(ss * (1.f / D) + a.eps);
  float y[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) y[i] = o[i] * inv * w[i] / (1.f + exp_fast(-g[i]));
  st8(static_cast<O*>(a.out) + off, y);
}

template <int D>
hipError_t launch_d(const NormLaunch& s, const NormArgs& a, hipStream_t stream) {
  const int64_t threads = a.rows * (D / 8);
  const unsigned blocks = static_cast<unsigned>((threads + NTN - 1) / NTN);
  if (s.gate_bf16) {
    if (s.out_bf16) hipLaunchKernelGGL((gated_rmsnorm_kernel<D, bf16_t, bf16_t>), dim3(blocks), dim3(NTN), 0, stream, a);
    else hipLaunchKernelGGL((gated_rmsnorm_kernel<D, bf16_t, float>), dim3(blocks), dim3(NTN), 0, stream, a);
  } else {
    if (s.out_bf16) hipLaunchKernelGGL((gated_rmsnorm_kernel<D, float, bf16_t>), dim3(blocks), dim3(NTN), 0, stream, a);
    else hipLaunchKernelGGL((gated_rmsnorm_kernel<D, float, float>), dim3(blocks), dim3(NTN), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gated_rmsnorm(const NormLaunch& s, hipStream_t stream) {
  if (s.rows == 0) return hipSuccess;
  NormArgs a{s.o, s.gate, s.weight, s.out, s.rows, s.eps};
  switch (s.d) {
    case 16: return launch_d<16>(s, a, stream);
    case 32: return launch_d<32>(s, a, stream);
    case 64: return launch_d<64>(s, a, stream);
    case 128: return launch_d<128>(s, a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kda
