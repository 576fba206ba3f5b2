// Device-side helpers shared by the HIP kernels of libqfa (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qfa.h"
#include "qfa_index.h"

namespace qfa {

typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
  return __uint_as_float(b16 << 16);
}

__device__ __forceinline__ float f16_bits_to_f32(uint32_t h16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)h16);
  return (float)h;
}

// Round a float to bf16 (nearest-even; inputs are finite) and return the bits.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
  _Float16 h = (_Float16)f;
  return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

// Load a scale stored as fp32 or fp16 without reading past its own bytes:
// two 16-bit loads (for fp16 both read the scale itself; for fp32 they read
// its low and high halves) and a select, no branch. A branch around a load
// makes the compiler wait for it, and for every load issued before it, at the
// merge point.
__device__ __forceinline__ float load_scale(const void* p, long idx, bool f16) {
  const uint16_t* h = (const uint16_t*)p;
  long i0, i1;
  ix::scale_halves(idx, f16, i0, i1);
  const uint32_t lo = h[i0], hi = h[i1];
  return f16 ? f16_bits_to_f32(lo) : __uint_as_float(lo | (hi << 16));
}

}  // namespace qfa
