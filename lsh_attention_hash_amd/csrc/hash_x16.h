// hash_x16.h -- the fp16 form of a bf16 qk row in the matrix-core hash and
// the bounds its certificate needs. Shared by the hash kernel (which converts
// the rows it loads), the hash's norm pre-pass and the projection kernel,
// which produces the same bounds for the rows it writes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {
namespace hx {

constexpr float kF16Max = 65504.0f;
constexpr float kF16MinNormal = 6.103515625e-05f;  // 2^-14

// fp16 value of a rotation entry: clamped to the fp16 range and flushed to 0
// below the smallest normal
__device__ __forceinline__ float f16_round(float x) {
  const float c = fminf(fmaxf(x, -kF16Max), kF16Max);
  return fabsf(c) < kF16MinNormal ? 0.f : (float)(_Float16)c;
}

// fp16 values of the bf16 pair in w (low half first) as the projection uses
// them: converted toward zero by v_cvt_pkrtz_f16_f32, exactly for every bf16
// value in the fp16 range, within 2^-24 below it (fp16 subnormals, which the
// matrix cores and v_dot2 take as they are), to the largest finite fp16
// value above it. Every kernel that makes or bounds the fp16 row uses this.
__device__ __forceinline__ uint32_t x16_pair(uint32_t w, float& x0, float& x1) {
  x0 = __uint_as_float(w << 16);
  x1 = __uint_as_float(w & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(x0, x1));
}

// One 16-byte piece of a bf16 row (8 values): adds to b the squares of the
// conversion error of its fp16 form and to c the squares of the values.
// (|x16| <= |x| for every value, the conversion being toward zero, so the
// row's |x| bounds |x16|.)
__device__ __forceinline__ void x16_piece(uint4 raw, float& b, float& c) {
  const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float x0, x1;
    const uint32_t h = x16_pair(wv[q], x0, x1);
    c = fmaf(x0, x0, fmaf(x1, x1, c));
    const float h0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(h & 0xFFFFu));
    const float h1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(h >> 16));
    b = fmaf(x0 - h0, x0 - h0, fmaf(x1 - h1, x1 - h1, b));
  }
}

// upper bounds of |x16| and |x - x16| from the row's sums of x^2 (c) and of
// (x - x16)^2 (b), covering their fp32 rounding
__device__ __forceinline__ float2 norm_bounds(float c, float b) {
  return make_float2(sqrtf(c) * (1.0f + 1e-5f), sqrtf(b) * (1.0f + 1e-5f));
}

}  // namespace hx
}  // namespace lsh
