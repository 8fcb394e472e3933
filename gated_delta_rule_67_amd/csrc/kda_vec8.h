// kda_vec8.h -- 8 consecutive elements as fp32 registers, from and to fp32 or
// bf16 memory (bf16: one 16-byte access; stores round to nearest even from
// fp32, for finite values).  Used by the elementwise kernels.
#pragma once

#include "kda_common.h"

namespace kda {

__device__ __forceinline__ void load8f(const float* p, float (&o)[8]) {
  const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w; o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}
__device__ __forceinline__ void load8f(const bf16_t* p, float (&o)[8]) {
  const uint4 u = *reinterpret_cast<const uint4*>(p);
  o[0] = bf16_lo(u.x); o[1] = bf16_hi(u.x); o[2] = bf16_lo(u.y); o[3] = bf16_hi(u.y);
  o[4] = bf16_lo(u.z); o[5] = bf16_hi(u.z); o[6] = bf16_lo(u.w); o[7] = bf16_hi(u.w);
}
__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ void store8f(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8f(bf16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = bf16_rne_bits(v[0]) | (bf16_rne_bits(v[1]) << 16);
  u.y = bf16_rne_bits(v[2]) | (bf16_rne_bits(v[3]) << 16);
  u.z = bf16_rne_bits(v[4]) | (bf16_rne_bits(v[5]) << 16);
  u.w = bf16_rne_bits(v[6]) | (bf16_rne_bits(v[7]) << 16);
  *reinterpret_cast<uint4*>(p) = u;
}

}  // namespace kda
