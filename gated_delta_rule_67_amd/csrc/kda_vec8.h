// kda_vec8.h -- 8 consecutive elements as fp32 registers, from and to fp32 or
// bf16 memory (bf16: one 16-byte access; stores round fp32 to nearest even in
// hardware, two values per instruction).  Used by the elementwise kernels.
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
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// two values rounded to nearest even as packed bf16 (one v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b) {
  bf16x2_t r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ void store8f(float* p, const float (&v)[8]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
  *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
}
__device__ __forceinline__ void store8f(bf16_t* p, const float (&v)[8]) {
  uint4 u;
  u.x = bf16_pack2(v[0], v[1]);
  u.y = bf16_pack2(v[2], v[3]);
  u.z = bf16_pack2(v[4], v[5]);
  u.w = bf16_pack2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = u;
}

}  // namespace kda
