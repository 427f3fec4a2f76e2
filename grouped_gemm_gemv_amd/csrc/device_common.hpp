// Device helpers shared by the HIP kernels of libmoe (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

// fp32 -> bf16, round to nearest, ties to even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return ((u >> 16) | 0x40u) & 0xffffu;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Element traits.  Every operand is moved in 16-byte chunks per lane; EPC is
// the number of elements in one chunk.
struct TBF16 {
  using T = uint16_t;
  static constexpr int EPC = 8;
};
struct TF32 {
  using T = float;
  static constexpr int EPC = 4;
};

// acc[16x16] += Wchunk (rows: 16 lanes' rows) x Achunk^T (cols: 16 lanes' rows).
//
// Operand placement (same for both element types): lane l supplies row
// (l % 16) of each operand, and the 16-byte chunk at byte offset 16*(l/16) of
// a 64-byte K slab.  The accumulator lane l holds output rows 4*(l/16)+r,
// r = 0..3, of column l % 16.  The K elements of one slab may be assigned to
// MFMA k-slots in any order as long as both operands use the same order:
//  - bf16: one v_mfma_f32_16x16x32_bf16 consumes the 8 bf16 of each chunk;
//  - fp32: four v_mfma_f32_16x16x4_f32, the q-th taking element q of each
//    lane's chunk (so MFMA q covers K positions {4*(l/16) + q}).
template <class Tr>
__device__ __forceinline__ f32x4_t mma16(const uint4& w, const uint4& a, f32x4_t acc);

template <>
__device__ __forceinline__ f32x4_t mma16<TBF16>(const uint4& w, const uint4& a, f32x4_t acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, w),
                                                 __builtin_bit_cast(bf16x8_t, a), acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ f32x4_t mma16<TF32>(const uint4& w, const uint4& a, f32x4_t acc) {
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.x), __uint_as_float(a.x), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.y), __uint_as_float(a.y), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.z), __uint_as_float(a.z), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(w.w), __uint_as_float(a.w), acc, 0, 0, 0);
  return acc;
}

// Store 4 consecutive outputs (fp32 values) in the element type.
template <class Tr>
__device__ __forceinline__ void store4(void* dst, float v0, float v1, float v2, float v3);

template <>
__device__ __forceinline__ void store4<TBF16>(void* dst, float v0, float v1, float v2, float v3) {
  uint2 o;
  o.x = f32_to_bf16(v0) | (f32_to_bf16(v1) << 16);
  o.y = f32_to_bf16(v2) | (f32_to_bf16(v3) << 16);
  *reinterpret_cast<uint2*>(dst) = o;
}

template <>
__device__ __forceinline__ void store4<TF32>(void* dst, float v0, float v1, float v2, float v3) {
  *reinterpret_cast<float4*>(dst) = make_float4(v0, v1, v2, v3);
}

// Widen a 16-byte chunk to EPC fp32 values.
template <class Tr>
__device__ __forceinline__ void widen(const uint4& c, float* v);

template <>
__device__ __forceinline__ void widen<TBF16>(const uint4& c, float* v) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <>
__device__ __forceinline__ void widen<TF32>(const uint4& c, float* v) {
  v[0] = __uint_as_float(c.x);
  v[1] = __uint_as_float(c.y);
  v[2] = __uint_as_float(c.z);
  v[3] = __uint_as_float(c.w);
}

// Narrow EPC fp32 values to one 16-byte chunk (bf16: round to nearest even).
template <class Tr>
__device__ __forceinline__ uint4 narrow(const float* v);

template <>
__device__ __forceinline__ uint4 narrow<TBF16>(const float* v) {
  uint4 c;
  c.x = f32_to_bf16(v[0]) | (f32_to_bf16(v[1]) << 16);
  c.y = f32_to_bf16(v[2]) | (f32_to_bf16(v[3]) << 16);
  c.z = f32_to_bf16(v[4]) | (f32_to_bf16(v[5]) << 16);
  c.w = f32_to_bf16(v[6]) | (f32_to_bf16(v[7]) << 16);
  return c;
}

template <>
__device__ __forceinline__ uint4 narrow<TF32>(const float* v) {
  return make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3]));
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (lane == 0) ? 0ull : (~0ull >> (64 - lane)); }

}  // namespace moe
