// hash_x16.h -- the per-row preparation of the matrix-core hash: the fp16
// copy of a bf16 qk row and the bounds the hash's certificate needs. Shared
// by the hash's own pre-pass and by the projection kernel, which produces the
// same values for the rows it writes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {
namespace hx {

constexpr float kF16Max = 65504.0f;
constexpr float kF16MinNormal = 6.103515625e-05f;  // 2^-14

// fp16 value of x as the projection uses it: clamped to the fp16 range and
// flushed to 0 below the smallest normal
__device__ __forceinline__ float f16_round(float x) {
  const float c = fminf(fmaxf(x, -kF16Max), kF16Max);
  return fabsf(c) < kF16MinNormal ? 0.f : (float)(_Float16)c;
}

// One 16-byte piece of a bf16 row (8 values): returns its fp16 copy and adds
// to a, b, c the squares of the copy, of the rounding error and of the values.
__device__ __forceinline__ uint4 x16_piece(uint4 raw, float& a, float& b, float& c) {
  const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
  uint32_t out[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x0 = __uint_as_float(wv[q] << 16), x1 = __uint_as_float(wv[q] & 0xFFFF0000u);
    c = fmaf(x0, x0, fmaf(x1, x1, c));
    const float h0 = f16_round(x0), h1 = f16_round(x1);
    const _Float16 e0 = (_Float16)h0, e1 = (_Float16)h1;
    out[q] = (uint32_t)__builtin_bit_cast(uint16_t, e0) |
             ((uint32_t)__builtin_bit_cast(uint16_t, e1) << 16);
    a = fmaf(h0, h0, fmaf(h1, h1, a));
    b = fmaf(x0 - h0, x0 - h0, fmaf(x1 - h1, x1 - h1, b));
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// upper bounds of |x16| and |x - x16| from the row's sums (covering their
// fp32 rounding)
__device__ __forceinline__ float2 norm_bounds(float a, float b) {
  return make_float2(sqrtf(a) * (1.0f + 1e-5f), sqrtf(b) * (1.0f + 1e-5f));
}

}  // namespace hx
}  // namespace lsh
