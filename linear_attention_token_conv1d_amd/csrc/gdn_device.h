// Device helpers shared by the gfx950 kernels: bf16 <-> fp32 conversion,
// 16-byte vector loads/stores, wave64 DPP reductions and MFMA fragments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- scalars

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  f32x2 v = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float to_f32(__bf16 v) { return (float)v; }
__device__ __forceinline__ float to_f32(float v) { return v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ __bf16 from_f32<__bf16>(float v) { return (__bf16)v; }

// ------------------------------------------------------ 8-element vectors
// load8/store8 move 8 consecutive elements (16 B of bf16, 32 B of fp32);
// the pointer must be aligned to the vector size.

__device__ __forceinline__ void load8(const __bf16* p, float (&v)[8]) {
  uint4 w = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8(const float* p, float (&v)[8]) {
  float4 a = reinterpret_cast<const float4*>(p)[0];
  float4 b = reinterpret_cast<const float4*>(p)[1];
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}
__device__ __forceinline__ void store8(__bf16* p, const float (&v)[8]) {
  uint4 w;
  w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
  *reinterpret_cast<uint4*>(p) = w;
}
__device__ __forceinline__ void store8(float* p, const float (&v)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(v[0], v[1], v[2], v[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(v[4], v[5], v[6], v[7]);
}
// 4-element variants (8 B of bf16, 16 B of fp32).
__device__ __forceinline__ void load4(const __bf16* p, float (&v)[4]) {
  uint2 w = *reinterpret_cast<const uint2*>(p);
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
}
__device__ __forceinline__ void load4(const float* p, float (&v)[4]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
}
__device__ __forceinline__ void store4(__bf16* p, const float (&v)[4]) {
  uint2 w;
  w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
  *reinterpret_cast<uint2*>(p) = w;
}
__device__ __forceinline__ void store4(float* p, const float (&v)[4]) {
  *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
}

// Variants for data touched once per launch (the decode state):
// nontemporal stores; nontemporal loads for fp32 rows and ordinary loads for
// bf16 rows, each the faster on the 27B decode shape (bf16 state 146 against
// 150 us a step; fp32 state 311 against 335).
typedef unsigned gdn_u4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void load8_stream(const __bf16* p, float (&v)[8]) {
  const gdn_u4 w = *(reinterpret_cast<const gdn_u4*>(p));
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
  v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
  v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
  v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
}
__device__ __forceinline__ void load8_stream(const float* p, float (&v)[8]) {
  const gdn_u4 a = __builtin_nontemporal_load(reinterpret_cast<const gdn_u4*>(p));
  const gdn_u4 b = __builtin_nontemporal_load(reinterpret_cast<const gdn_u4*>(p) + 1);
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z);
  v[3] = __uint_as_float(a.w); v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
  v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
}
__device__ __forceinline__ void store8_stream(__bf16* p, const float (&v)[8]) {
  gdn_u4 w;
  w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
  w.z = pack_bf16x2(v[4], v[5]); w.w = pack_bf16x2(v[6], v[7]);
  __builtin_nontemporal_store(w, reinterpret_cast<gdn_u4*>(p));
}
__device__ __forceinline__ void store8_stream(float* p, const float (&v)[8]) {
  gdn_u4 a, b;
  a.x = __float_as_uint(v[0]); a.y = __float_as_uint(v[1]); a.z = __float_as_uint(v[2]);
  a.w = __float_as_uint(v[3]); b.x = __float_as_uint(v[4]); b.y = __float_as_uint(v[5]);
  b.z = __float_as_uint(v[6]); b.w = __float_as_uint(v[7]);
  __builtin_nontemporal_store(a, reinterpret_cast<gdn_u4*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<gdn_u4*>(p) + 1);
}
__device__ __forceinline__ void load4_stream(const __bf16* p, float (&v)[4]) {
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  const u2 w = *(reinterpret_cast<const u2*>(p));
  v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
}
__device__ __forceinline__ void load4_stream(const float* p, float (&v)[4]) {
  const gdn_u4 a = __builtin_nontemporal_load(reinterpret_cast<const gdn_u4*>(p));
  v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z);
  v[3] = __uint_as_float(a.w);
}
__device__ __forceinline__ void store4_stream(__bf16* p, const float (&v)[4]) {
  typedef unsigned u2 __attribute__((ext_vector_type(2)));
  u2 w;
  w.x = pack_bf16x2(v[0], v[1]); w.y = pack_bf16x2(v[2], v[3]);
  __builtin_nontemporal_store(w, reinterpret_cast<u2*>(p));
}
__device__ __forceinline__ void store4_stream(float* p, const float (&v)[4]) {
  gdn_u4 a;
  a.x = __float_as_uint(v[0]); a.y = __float_as_uint(v[1]); a.z = __float_as_uint(v[2]);
  a.w = __float_as_uint(v[3]);
  __builtin_nontemporal_store(a, reinterpret_cast<gdn_u4*>(p));
}

// ---------------------------------------------------------- reductions
// DPP controls (GCN/CDNA encoding).
enum : int {
  DPP_QUAD_1032 = 0xB1,      // quad_perm [1,0,3,2]: partner lane ^ 1
  DPP_QUAD_2301 = 0x4E,      // quad_perm [2,3,0,1]: partner lane ^ 2
  DPP_ROW_MIRROR = 0x140,    // lane i <- lane 15 - i within a row of 16
  DPP_ROW_HALF_MIRROR = 0x141  // lane i <- lane 7 - i within a half row of 8
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

// Sum over each group of 16 consecutive lanes; every lane receives its group's sum.
__device__ __forceinline__ float row16_sum(float v) {
  v += dpp_f32<DPP_QUAD_1032>(v);
  v += dpp_f32<DPP_QUAD_2301>(v);
  v += dpp_f32<DPP_ROW_HALF_MIRROR>(v);
  v += dpp_f32<DPP_ROW_MIRROR>(v);
  return v;
}

// Sum over the whole wave of 64 lanes; every lane receives the sum.
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

// y * sigmoid(y) with a reciprocal-based divide (within a few ulp; 0 for
// very negative y, where 1 + e^-y overflows and the reciprocal is 0)
__device__ __forceinline__ float silu(float y) { return __fdividef(y, 1.0f + __expf(-y)); }

// Index arrays a kernel only reads (chunk offsets, cu_seqlens, state slots)
// are never written while it runs; reading them through the constant
// address space lets loads at uniform indices go through the scalar cache.
typedef const __attribute__((address_space(4))) int32_t cint32;
__device__ __forceinline__ cint32* as_const(const int32_t* p) { return (cint32*)p; }

}  // namespace gdn
