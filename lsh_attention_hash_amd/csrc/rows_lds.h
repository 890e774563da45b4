// rows_lds.h -- staging one 64-row chunk of bf16 rows (gathered through a
// permutation) into LDS for the matrix-core kernels, row-major and by pairs
// of 4-row groups.
//
// Row-major rows (+16-byte pad) give a product over dims its operands: lane l
// reads 16 bytes of row l % 16. The pair layout gives a product over rows its
// A operand: group a (rows 4a .. 4a+3) and group a + 4 form pair
// (a % 4) + 4 (a / 8); per dim 16 bytes hold the 4 rows of group a, then the
// 4 rows of group a + 4, and a 16-byte pad follows every 8 dims. A 256-thread
// workgroup loads a chunk with whole 256-byte rows per load instruction.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {
namespace rows {

constexpr int kChunk = 64;
constexpr int kThreads = 256;

template <int D>
struct BLay {
  static constexpr int kSegs = D / 8;               // 16-byte pieces per row
  static constexpr int kRow = D * 2 + 16;           // row-major stride (bytes, +16 pad)
  static constexpr int kBlk8 = 8 * 16 + 16;         // 8 dims of a group pair (+16 pad)
  static constexpr int kPair = D / 8 * kBlk8;       // one pair of 4-row groups
  static constexpr int kRM = kChunk * kRow;         // a chunk, row-major
  static constexpr int kPM = kChunk / 8 * kPair;    // a chunk, by group pairs
  static constexpr int kUsers = (kChunk / 4) * kSegs;  // (group, piece) loaders
  static_assert(kUsers <= kThreads, "one group piece per thread");
};

// Thread t < kUsers loads piece t % kSegs of the 4 rows of group t / kSegs
// (rows at the positions pn[] of a chunk, from rows of `D` bf16 at `base`).
template <int D>
__device__ __forceinline__ void load_group(uint4* r, const unsigned char* base, const int* pn) {
  using Lay = BLay<D>;
  const int t = threadIdx.x;
  if (t < Lay::kUsers) {
    const int qd = t / Lay::kSegs, sg = t % Lay::kSegs;
    const int4 p4 = *(const int4*)(pn + 4 * qd);
    const int pos[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = *(const uint4*)(base + (int64_t)pos[k] * (D * 2) + sg * 16);
  }
}

// the same registers, row-major
template <int D>
__device__ __forceinline__ void store_rm(unsigned char* dst, const uint4* r) {
  using Lay = BLay<D>;
  const int t = threadIdx.x;
  if (t < Lay::kUsers) {
    const int qd = t / Lay::kSegs, sg = t % Lay::kSegs;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint4 x = r[k];
      asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
      *(uint4*)(dst + (4 * qd + k) * Lay::kRow + sg * 16) = x;
    }
  }
}

// the same registers by group pairs: group qd is half (qd / 4) % 2 of pair
// (qd % 4) + 4 (qd / 8); per dim 8 bytes of its 4 rows
template <int D>
__device__ __forceinline__ void store_pair(unsigned char* dst, const uint4* r) {
  using Lay = BLay<D>;
  const int t = threadIdx.x;
  if (t < Lay::kUsers) {
    const int qd = t / Lay::kSegs, sg = t % Lay::kSegs;
    const int pair = (qd & 3) + 4 * (qd >> 3), half = (qd >> 2) & 1;
    unsigned char* d = dst + pair * Lay::kPair + sg * Lay::kBlk8 + half * 8;
    const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
    const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
    const uint32_t w2[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
    const uint32_t w3[4] = {r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *(uint2*)(d + 32 * u) =
          make_uint2((w0[u] & 0xFFFFu) | (w1[u] << 16), (w2[u] & 0xFFFFu) | (w3[u] << 16));
      *(uint2*)(d + 32 * u + 16) = make_uint2((w0[u] >> 16) | (w1[u] & 0xFFFF0000u),
                                              (w2[u] >> 16) | (w3[u] & 0xFFFF0000u));
    }
  }
}

__device__ __forceinline__ void zero_lds(unsigned char* p, int bytes) {
  for (int i = threadIdx.x; i < bytes / 16; i += kThreads) ((uint4*)p)[i] = uint4{};
}

}  // namespace rows
}  // namespace lsh
