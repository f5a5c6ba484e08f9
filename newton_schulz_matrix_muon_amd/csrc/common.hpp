// Shared device helpers for the gfx950 kernels: element types and loads/stores by runtime
// dtype.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mns {

enum Dtype : int { F32 = 0, BF16 = 1, F16 = 2 };

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__host__ __device__ inline int dtype_size(int dt) { return dt == F32 ? 4 : 2; }

// fp32 -> bf16, round to nearest even, NaN kept quiet with its upper payload bits: gfx950's
// v_cvt_pk_bf16_f32, which gives exactly the bits of the bitwise definition
// ((u + 0x7fff + lsb) >> 16, NaN -> (u >> 16) | 0x40) for every one of the 2^32 inputs.
__device__ inline uint16_t f32_to_bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ inline float bf16_bits_to_f32(uint16_t h) { return __uint_as_float(((uint32_t)h) << 16); }

__device__ inline uint16_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;  // hardware conversion, round-to-nearest-even
  return __builtin_bit_cast(uint16_t, h);
}

__device__ inline float f16_bits_to_f32(uint16_t h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// Two fp32 values -> two packed 16-bit values (lo in bits 0..15) with one packed conversion
// (v_cvt_pk_bf16_f32 / v_cvt_pk_f16_f32; same rounding as the scalar conversions above).
template <typename H>
__device__ inline uint32_t pack2(float lo, float hi) {
  typedef float f32x2 __attribute__((ext_vector_type(2)));
  typedef H h16x2 __attribute__((ext_vector_type(2)));
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, h16x2));
}

// Load element `idx` of a buffer of runtime dtype `dt` as fp32.
__device__ inline float load_elem(const void* p, int dt, int64_t idx) {
  if (dt == F32) return reinterpret_cast<const float*>(p)[idx];
  uint16_t h = reinterpret_cast<const uint16_t*>(p)[idx];
  return dt == BF16 ? bf16_bits_to_f32(h) : f16_bits_to_f32(h);
}

// Store fp32 `v` into element `idx` of a buffer of runtime dtype `dt` (RNE rounding).
__device__ inline void store_elem(void* p, int dt, int64_t idx, float v) {
  if (dt == F32) {
    reinterpret_cast<float*>(p)[idx] = v;
  } else {
    reinterpret_cast<uint16_t*>(p)[idx] = dt == BF16 ? f32_to_bf16_bits(v) : f32_to_f16_bits(v);
  }
}

}  // namespace mns
