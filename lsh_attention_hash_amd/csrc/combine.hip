// combine.hip -- logsumexp-weighted combination of the hash rounds.
//
// The multi-round section of the Reformer summary (p2.ttnews.xyz) leaves the
// combination to the original paper. Reading taken: out(i) is the softmax
// over rounds of lse_r(i) applied to the per-round outputs,
//   w_r = exp(lse_r - max_r lse_r) / sum_r' exp(lse_r' - max_r lse_r'),
//   out(i) = sum_r w_r o_r(i),
// which equals one softmax over the multiset union of all rounds' windows.
// The per-round rows are already at original positions (the attention kernel
// scatters them), so this kernel streams them in order.
#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

__device__ __forceinline__ float ld_f32(const float* p) { return *p; }
__device__ __forceinline__ float ld_f32(const _Float16* p) { return (float)*p; }

template <typename OutT, typename OT>
__global__ __launch_bounds__(256) void k_combine(const OT* __restrict__ o,
                                                 const float* __restrict__ lse,
                                                 OutT* __restrict__ out, int L, int R, int d,
                                                 int64_t n_rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
       row < n_rows; row += waves) {
    const int64_t bh = row / L;
    const int64_t i = row - bh * L;
    const float* lr = lse + bh * R * L + i;
    float mx = -INFINITY;
    for (int r = 0; r < R; ++r) mx = fmaxf(mx, lr[(int64_t)r * L]);
    float sum = 0.f;
    for (int r = 0; r < R; ++r) sum += __expf(lr[(int64_t)r * L] - mx);
    const float inv_sum = 1.0f / sum;
    for (int u = lane; u < d; u += kWave) {
      float acc = 0.f;
      for (int r = 0; r < R; ++r) {
        const float w = __expf(lr[(int64_t)r * L] - mx) * inv_sum;
        acc += w * ld_f32(o + ((bh * R + r) * L + i) * d + u);
      }
      out[row * d + u] = from_f32<OutT>(acc);
    }
  }
}

template <typename OT>
void launch_t(const Problem& p, const OT* o, const float* lse, void* out, hipStream_t s) {
  const int64_t n = p.n_token_heads();
  const int64_t want = (n + 3) / 4;
  const unsigned blocks = (unsigned)(want < 131072 ? want : 131072);
  if (p.out_dtype == LSH_ATTN_BF16)
    hipLaunchKernelGGL((k_combine<bf16_t, OT>), dim3(blocks), dim3(256), 0, s, o, lse,
                       (bf16_t*)out, p.L, p.R, p.d, n);
  else
    hipLaunchKernelGGL((k_combine<float, OT>), dim3(blocks), dim3(256), 0, s, o, lse,
                       (float*)out, p.L, p.R, p.d, n);
}

}  // namespace

hipError_t launch_combine(const Problem& p, const void* o, bool o_half, const float* lse,
                          void* out, hipStream_t s) {
  if (o_half) launch_t<_Float16>(p, (const _Float16*)o, lse, out, s);
  else launch_t<float>(p, (const float*)o, lse, out, s);
  return hipGetLastError();
}

}  // namespace lsh
