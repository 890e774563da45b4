// hash.hip -- random-rotation LSH bucket ids.
//
// Reformer summary (p2.ttnews.xyz), section on LSH: with R of size
// [d, n_buckets/2], h(x) = argmax([xR; -xR]); multi-round section: one
// independent R per round. Ties go to the lowest index of the concatenation.
//
// This file holds the exact kernel: each wave owns one (segment, position)
// row and every lane projects a strided subset of the n_buckets/2 columns in
// fp64. The products of a bf16 or fp32 input with an fp32 rotation are exact
// in fp64, and the sum runs over t = 0..d-1 in order, so the projection is the
// correctly ordered fp64 sum and the decision is the fp64 argmax.
#include <float.h>
#include <limits.h>

#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

// Better of two (value, index) candidates under "largest value, lowest index".
__device__ __forceinline__ void take_better(double& v, int& k, double ov, int ok) {
  if (ov > v || (ov == v && ok < k)) {
    v = ov;
    k = ok;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void k_hash_exact(const T* __restrict__ qk,
                                                    const float* __restrict__ rot,
                                                    uint16_t* __restrict__ buckets,
                                                    int32_t* __restrict__ buckets_out, int L,
                                                    int d, int half, int R, int64_t n_rows) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / kWave);
  for (int64_t row = (int64_t)blockIdx.x * (blockDim.x / kWave) + (threadIdx.x / kWave);
       row < n_rows; row += waves) {
    const int64_t seg = row / L;
    const int64_t i = row - seg * L;
    const int64_t bh = seg / R;
    const int r = (int)(seg - bh * R);
    const T* x = qk + (bh * L + i) * d;
    const float* Rr = rot + (int64_t)r * d * half;
    double best = -DBL_MAX;
    int bidx = INT_MAX;
    for (int k = lane; k < half; k += kWave) {
      double p = 0.0;
      for (int t = 0; t < d; ++t) p += (double)to_f32(x[t]) * (double)Rr[(int64_t)t * half + k];
      take_better(best, bidx, p, k);          // entry k of [xR; -xR]
      take_better(best, bidx, -p, k + half);  // entry k + half
    }
    for (int off = kWave / 2; off > 0; off >>= 1) {
      const double ov = __shfl_xor(best, off);
      const int ok = __shfl_xor(bidx, off);
      take_better(best, bidx, ov, ok);
    }
    // NaN inputs leave no candidate; keep the id in range so the sort still
    // produces a permutation (results are undefined for such inputs anyway).
    if (bidx < 0 || bidx >= 2 * half) bidx = 0;
    if (lane == 0) {
      buckets[row] = (uint16_t)bidx;
      if (buckets_out) buckets_out[row] = bidx;
    }
  }
}

__global__ void k_fill_bucket0(uint16_t* __restrict__ buckets, int32_t* __restrict__ buckets_out,
                               int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x) {
    buckets[i] = 0;
    if (buckets_out) buckets_out[i] = 0;
  }
}

}  // namespace

hipError_t launch_hash_exact(const Problem& p, const void* qk, const float* rot,
                             uint16_t* buckets, int32_t* buckets_out, hipStream_t s) {
  const int64_t n = p.n_rows();
  if (p.nb == 1) {
    const int64_t blocks = (n + 255) / 256 < 65536 ? (n + 255) / 256 : 65536;
    hipLaunchKernelGGL(k_fill_bucket0, dim3((unsigned)blocks), dim3(256), 0, s, buckets,
                       buckets_out, n);
    return hipGetLastError();
  }
  const int64_t want = (n + 3) / 4;
  const unsigned blocks = (unsigned)(want < 262144 ? want : 262144);
  if (p.dtype == LSH_ATTN_BF16)
    hipLaunchKernelGGL(k_hash_exact<bf16_t>, dim3(blocks), dim3(256), 0, s,
                       (const bf16_t*)qk, rot, buckets, buckets_out, p.L, p.d, p.half(), p.R, n);
  else
    hipLaunchKernelGGL(k_hash_exact<float>, dim3(blocks), dim3(256), 0, s, (const float*)qk,
                       rot, buckets, buckets_out, p.L, p.d, p.half(), p.R, n);
  return hipGetLastError();
}

}  // namespace lsh
