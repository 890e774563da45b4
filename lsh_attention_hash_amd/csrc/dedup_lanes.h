// dedup_lanes.h -- the de-duplicated reading's count on matrix-core kernels:
// N_ij, the number of rounds whose window (and bucket, with the same-bucket
// mask) gives key j to query i (Reformer, www.2kiu.com/news/5253576/, section
// 2.2: a key that several rounds give a query counts once, so each logit is
// lowered by log N_ij).
//
// Each row carries u16 lanes: its chunk (mod 2^16) in each of up to 8 rounds,
// two rounds per 32-bit word, and its bucket in each round. A key's lanes past
// R hold chunk 0x8000, a query's hold 0, so they never match. The count takes
// the chunk difference d = chunk_key - chunk_query per round: the key is in the
// window when d + 1 <= 1 (2 with the look-ahead), computed as a saturating
// subtraction that is 0 exactly then; a bucket mismatch makes the lane nonzero
// too; the nonzero lanes are the rounds that do not give the pair.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {
namespace dedup {

constexpr int kMaxRounds = 8;
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

// The lanes of the row at position pos of one (batch, head): inv_bh and bk_bh
// are [R, L] (the sorted slot of each position, and its bucket, per round);
// bk_bh is read only with the same-bucket mask. Key form (lanes past R 0x8000).
__device__ __forceinline__ void row_lanes(const int32_t* inv_bh, const uint16_t* bk_bh, int R,
                                          int L, int m, int pos, bool sb, uint32_t (&cw)[4],
                                          uint32_t (&bw)[4]) {
#pragma unroll
  for (int u = 0; u < kMaxRounds; u += 2) {
    uint32_t c = 0x80008000u, b = 0u;
#pragma unroll
    for (int h = 0; h < 2; ++h)
      if (u + h < R) {
        const int64_t o = (int64_t)(u + h) * L + pos;
        const uint32_t cc = (uint32_t)(inv_bh[o] / m) & 0xFFFFu;
        c = (c & ~(0xFFFFu << (16 * h))) | (cc << (16 * h));
        if (sb) b |= (uint32_t)bk_bh[o] << (16 * h);
      }
    cw[u / 2] = c;
    bw[u / 2] = b;
  }
}

// a row's key lanes in query form (chunk lanes past R set to 0)
__device__ __forceinline__ void query_lanes(const uint32_t (&kc)[4], int R, uint32_t (&qc)[4]) {
#pragma unroll
  for (int k = 0; k < kMaxRounds / 2; ++k) {
    const uint32_t keep = 2 * k + 1 < R ? 0xFFFFFFFFu : (2 * k < R ? 0xFFFFu : 0u);
    qc[k] = kc[k] & keep;
  }
}

// log2 N_ij from the query's lanes (qc, qb) and the key's (kc, kb)
__device__ __forceinline__ float log2_rounds(const uint32_t (&qc)[4], const uint32_t (&qb)[4],
                                             const uint32_t (&kc)[4], const uint32_t (&kb)[4],
                                             int R, bool la, bool sb) {
  const unsigned short lim = la ? 2 : 1;
  const u16x2_t one2 = {1, 1}, lim2 = {lim, lim};
  uint32_t out = 0u;
  int lanes = 0;
#pragma unroll
  for (int k = 0; k < kMaxRounds / 2; ++k) {
    if (2 * k >= R) break;
    const u16x2_t d = __builtin_bit_cast(u16x2_t, kc[k]) - __builtin_bit_cast(u16x2_t, qc[k]);
    u16x2_t y = __builtin_elementwise_sub_sat(d + one2, lim2);
    if (sb) y |= __builtin_bit_cast(u16x2_t, kb[k] ^ qb[k]);
    y = __builtin_elementwise_min(y, one2);
    out = __builtin_amdgcn_udot2(y, one2, out, false);
    lanes += 2;
  }
  return __log2f((float)max(lanes - (int)out, 1));
}

}  // namespace dedup
}  // namespace lsh
