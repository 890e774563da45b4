// gather.hip -- qk and v rows copied into sorted order, per round.
//
// The sorted sequence of the Reformer summary's LSH-attention section made
// explicit: qk_sorted[seg][s] = qk[b][h][perm[s]], and the same for v. Each
// row is d contiguous elements, copied in 16-byte pieces (rows are 16-byte
// aligned: d * element size is a multiple of 16 and the base pointers are
// checked by the host code).
#include "internal.h"

namespace lsh {
namespace {

__global__ __launch_bounds__(256) void k_gather(const uint4* __restrict__ qk,
                                                const uint4* __restrict__ v,
                                                const int32_t* __restrict__ perm,
                                                uint4* __restrict__ qk_s, uint4* __restrict__ v_s,
                                                int L, int R, int pieces, int64_t n_rows) {
  const int64_t total = n_rows * pieces;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = g / pieces;
    const int piece = (int)(g - row * pieces);
    const int64_t seg = row / L;
    const int64_t bh = seg / R;
    const int64_t src = (bh * L + perm[row]) * pieces + piece;
    qk_s[g] = qk[src];
    v_s[g] = v[src];
  }
}

}  // namespace

hipError_t launch_gather(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                         void* qk_sorted, void* v_sorted, hipStream_t s) {
  const int esize = p.dtype == LSH_ATTN_BF16 ? 2 : 4;
  const int pieces = p.d * esize / 16;
  const int64_t total = p.n_rows() * pieces;
  const int64_t want = (total + 255) / 256;
  const unsigned blocks = (unsigned)(want < 262144 ? want : 262144);
  hipLaunchKernelGGL(k_gather, dim3(blocks), dim3(256), 0, s, (const uint4*)qk, (const uint4*)v,
                     perm, (uint4*)qk_sorted, (uint4*)v_sorted, p.L, p.R, pieces, p.n_rows());
  return hipGetLastError();
}

}  // namespace lsh
