// Device-side helpers shared by the gfx950 kernels: element types, 16-byte
// vector views, float <-> 16-bit conversions (round to nearest even), and the
// MFMA wrappers.  Written for CDNA4 wave64 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: non-temporal hint).
#ifndef PA_STREAM_NONTEMPORAL
#define PA_STREAM_NONTEMPORAL 1
#endif
__device__ __forceinline__ uint4 load_stream16(const uint4* p) {
#if PA_STREAM_NONTEMPORAL
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
#else
  return *p;
#endif
}

// Storage element tags.  `bits` is the type moved through memory.
struct F32 {
  using bits = uint32_t;
  static constexpr int kBytes = 4;
};
struct F16 {
  using bits = uint16_t;
  static constexpr int kBytes = 2;
};
struct BF16 {
  using bits = uint16_t;
  static constexpr int kBytes = 2;
};

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays a quiet NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  _Float16 h = __builtin_bit_cast(_Float16, static_cast<uint16_t>(h16));
  return static_cast<float>(h);
}

__device__ __forceinline__ uint32_t f32_to_f16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

template <typename T>
__device__ __forceinline__ uint32_t to_storage(float f);
template <>
__device__ __forceinline__ uint32_t to_storage<BF16>(float f) { return f32_to_bf16_rne(f); }
template <>
__device__ __forceinline__ uint32_t to_storage<F16>(float f) { return f32_to_f16_rne(f); }
template <>
__device__ __forceinline__ uint32_t to_storage<F32>(float f) { return __float_as_uint(f); }

template <typename T>
__device__ __forceinline__ float from_storage(uint32_t b);
template <>
__device__ __forceinline__ float from_storage<BF16>(uint32_t b) { return bf16_to_f32(b); }
template <>
__device__ __forceinline__ float from_storage<F16>(uint32_t b) { return f16_to_f32(b); }
template <>
__device__ __forceinline__ float from_storage<F32>(uint32_t b) { return __uint_as_float(b); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats rounded to nearest even into one 32-bit pair (a in the low
// half); gfx950 converts both in one instruction.
template <typename T>
__device__ __forceinline__ uint32_t pack2(float a, float b);
template <>
__device__ __forceinline__ uint32_t pack2<BF16>(float a, float b) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  const b2 v = {static_cast<__bf16>(a), static_cast<__bf16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}
template <>
__device__ __forceinline__ uint32_t pack2<F16>(float a, float b) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  const h2 v = {static_cast<_Float16>(a), static_cast<_Float16>(b)};
  return __builtin_bit_cast(uint32_t, v);
}

// The 16-bit pair (1.0, 1.0).
template <typename T>
__device__ __forceinline__ constexpr uint32_t ones2();
template <>
__device__ __forceinline__ constexpr uint32_t ones2<BF16>() { return 0x3f803f80u; }
template <>
__device__ __forceinline__ constexpr uint32_t ones2<F16>() { return 0x3c003c00u; }

// 16x16x32 (16-bit inputs) and 16x16x16 MFMA on raw bit vectors.
template <typename T>
__device__ __forceinline__ f32x4_t mfma_k32(uint4 a, uint4 b, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma_k32<BF16>(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma_k32<F16>(uint4 a, uint4 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
}

template <typename T>
__device__ __forceinline__ f32x4_t mfma_k16(uint2 a, uint2 b, f32x4_t c);
template <>
__device__ __forceinline__ f32x4_t mfma_k16<BF16>(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4_t, a),
                                                   __builtin_bit_cast(s16x4_t, b), c, 0, 0, 0);
}
template <>
__device__ __forceinline__ f32x4_t mfma_k16<F16>(uint2 a, uint2 b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                               __builtin_bit_cast(f16x4_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ f32x4_t mfma_f32_k4(float a, float b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Packed dot of two 16-bit pairs accumulated in float32.
template <typename T>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c);
template <>
__device__ __forceinline__ float dot2<F16>(uint32_t a, uint32_t b, float c) {
  typedef _Float16 h2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2, a), __builtin_bit_cast(h2, b), c, false);
}
template <>
__device__ __forceinline__ float dot2<BF16>(uint32_t a, uint32_t b, float c) {
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(b2, a), __builtin_bit_cast(b2, b), c,
                                         false);
}

}  // namespace pa
