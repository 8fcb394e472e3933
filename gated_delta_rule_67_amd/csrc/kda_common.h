// kda_common.h -- small device helpers shared by the libkda kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Element types of q, k, v as they arrive in HBM.
struct bf16_t { uint16_t bits; };

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x.bits) << 16);
}
__device__ __forceinline__ float bf16_lo(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// Two fp32 values rounded to nearest even as packed bf16 (one
// v_cvt_pk_bf16_f32); the first value in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b) {
  bf16x2_t r;
  r[0] = static_cast<__bf16>(a);
  r[1] = static_cast<__bf16>(b);
  return __builtin_bit_cast(uint32_t, r);
}
// Four consecutive outputs (8-byte aligned) as fp32 or rounded bf16.
__device__ __forceinline__ void store_out4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<float4*>(p) = make_float4(a, b, c, d);
}
__device__ __forceinline__ void store_out4(bf16_t* p, float a, float b, float c, float d) {
  *reinterpret_cast<uint2*>(p) = make_uint2(bf16_pack2(a, b), bf16_pack2(c, d));
}

// exp(x) through the hardware base-2 exponential; exp(-inf) = 0.
__device__ __forceinline__ float exp_fast(float x) {
  return __builtin_amdgcn_exp2f(x * 1.4426950408889634f);
}

// 16-byte fp32 load / store with the nontemporal hint (data read or written
// once: keep it from displacing reused lines in the caches).
__device__ __forceinline__ float4 load4_stream(const float* p) {
  const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
  return make_float4(x[0], x[1], x[2], x[3]);
}
__device__ __forceinline__ void store4_stream(float* p, float4 v) {
  __builtin_nontemporal_store(f32x4{v.x, v.y, v.z, v.w}, reinterpret_cast<f32x4*>(p));
}

// Load 4 consecutive elements (16-byte aligned for fp32, 8-byte for bf16) as floats.
__device__ __forceinline__ float4 load4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 load4(const bf16_t* p) {
  const uint2 u = *reinterpret_cast<const uint2*>(p);
  return make_float4(bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y));
}

// Workgroup barrier that orders LDS only: outstanding global loads (a
// prefetch) and stores stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f32x4 mfma32(f16x8 a, f16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(f16x4 a, f16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f16x8 ld8(const f16* p) { return *reinterpret_cast<const f16x8*>(p); }
__device__ __forceinline__ f16x4 ld4(const f16* p) { return *reinterpret_cast<const f16x4*>(p); }
__device__ __forceinline__ f16x4 h4(f32x4 x) {
  f16x4 r;
  r[0] = (f16)x[0]; r[1] = (f16)x[1]; r[2] = (f16)x[2]; r[3] = (f16)x[3];
  return r;
}
__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// Raw buffer resource over [base, base + bytes) (CDNA buffer descriptor, no
// swizzle, stride 0): a lane whose access falls outside the range has its
// store dropped by the hardware, so partial tiles need no branch.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void buffer_store16(f32x4 x, __amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(i32x4, x), r, static_cast<int>(byte_off), 0, 0);
}
typedef int i32x2 __attribute__((ext_vector_type(2)));
// four fp32 values rounded to bf16, one 8-byte range-checked store
__device__ __forceinline__ void buffer_store8_bf16(f32x4 x, __amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  const i32x2 v = {static_cast<int>(bf16_pack2(x[0], x[1])), static_cast<int>(bf16_pack2(x[2], x[3]))};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, static_cast<int>(byte_off), 0, 0);
}
// Range-checked loads through the same descriptor: a lane whose access falls
// outside the range reads zeros.
__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(byte_off), 0, 0));
}
__device__ __forceinline__ float buffer_load_f32(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, static_cast<int>(byte_off), 0, 0));
}

}  // namespace kda
