// dtype.h -- storage-type helpers for the device code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {

// bf16 is carried as its raw 16-bit pattern.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
  return __uint_as_float((uint32_t)x.bits << 16);
}

// float -> bf16, round to nearest even (finite inputs).
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return bf16_t{(uint16_t)(u >> 16)};
}

template <typename T>
__device__ __forceinline__ T from_f32(float f);
template <>
__device__ __forceinline__ float from_f32<float>(float f) { return f; }
template <>
__device__ __forceinline__ bf16_t from_f32<bf16_t>(float f) { return f32_to_bf16(f); }

}  // namespace lsh
