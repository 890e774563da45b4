// walks.h -- how the grids of the chunked kernels map blocks and waves to
// work: the head-grouped range walk of the attention kernels (forward, its
// variants and the backward products), the sort's tile order, and the hash's
// persistent walk over token tiles. These are the index computations the
// kernels run, kept here so that a host program (tests/walks_check.hip) can
// run exactly the same code over whole grids and check that every unit of
// work is visited once and every index stays in range.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {
namespace walks {

// ---------------------------------------------------------------------------
// Range walk of the chunk kernels: nseg (batch, head, round) segments of
// nchunks chunks, cut into ranges of `per` consecutive chunks; the grid has
// nseg * ranges blocks, dealt in groups of group_segs segments (all rounds
// of a few heads) with the segments of a group interleaved, so the blocks in
// flight read the rows of few heads.
struct RangeShape {
  int per;         // chunks per block
  int ranges;      // ranges per segment
  int group_segs;  // segments per group
  int64_t blocks;  // grid size
};

// resident: blocks in flight the group size is chosen for
__host__ __device__ inline RangeShape range_shape(int nchunks, int64_t nseg, int R, int max_per,
                                                  int64_t resident) {
  RangeShape s;
  s.per = nchunks < max_per ? nchunks : max_per;
  s.ranges = (nchunks + s.per - 1) / s.per;
  int64_t heads = (resident + (int64_t)s.ranges * R - 1) / ((int64_t)s.ranges * R);
  if (heads < 1) heads = 1;
  int64_t group_segs = heads * R;
  if (group_segs > nseg) group_segs = nseg;
  s.group_segs = (int)group_segs;
  s.blocks = nseg * s.ranges;
  return s;
}

// block b -> (segment, range)
__host__ __device__ inline void range_block(unsigned b, int group_segs, int ranges, int nseg,
                                            int64_t& seg, int& range) {
  const int group = b / (unsigned)(group_segs * ranges);
  const int first = group * group_segs;
  const int gn = group_segs < nseg - first ? group_segs : nseg - first;
  const int inner = b - group * group_segs * ranges;
  seg = first + inner % gn;
  range = inner / gn;
}

// ---------------------------------------------------------------------------
// Sort tiles: the grid has tiles * nseg blocks, dealt to the 8 XCDs round-robin.
// When the segments split evenly, block b takes a tile of a segment s with
// s % 8 == b % 8, so all tiles of a segment run on one XCD and the
// partial-line permutation writes of neighbouring tiles meet in its L2.
constexpr int kXcds = 8;
__host__ __device__ inline void sort_block_tile(unsigned b, int tiles, int64_t nseg, int64_t& seg,
                                                int& tile) {
  if (nseg % kXcds == 0) {
    const unsigned k = b / kXcds;
    seg = (int64_t)(b % kXcds) + (int64_t)kXcds * (k / (unsigned)tiles);
    tile = (int)(k % (unsigned)tiles);
  } else {
    seg = b / (unsigned)tiles;
    tile = (int)(b % (unsigned)tiles);
  }
}

// ---------------------------------------------------------------------------
// Hash: a persistent grid of G = 8 R k workgroups. Workgroup b serves round
// r and token tiles j = grp, grp + G/R, ... (tiles of tok_wg consecutive
// token-heads), with b -> (xcd = b % 8, kk = b / 8, r = kk % R,
// grp = xcd + 8 (kk / R)): the R workgroups that read one token tile differ
// only in r and share an XCD.
__host__ __device__ inline void hash_block(unsigned b, int R, int& r, int& grp) {
  const int xcd = b & 7;
  const int kk = b >> 3;
  r = kk % R;
  grp = xcd + 8 * (kk / R);
}

// grid size: as many resident workgroups as fit (n_cu * per_cu), rounded
// down to a multiple of 8 R (at least 8 R), and no more than the token tiles
// need
__host__ __device__ inline int64_t hash_grid(int n_cu, int per_cu, int R, int n_tok_tiles) {
  const int unit = 8 * R;
  int64_t grid = (int64_t)n_cu * per_cu;
  grid = (grid / unit) * unit;
  if (grid < unit) grid = unit;
  const int64_t max_grid = (int64_t)unit * ((n_tok_tiles + 7) / 8);
  if (grid > max_grid) grid = max_grid;
  return grid;
}

// (head, position) of a wave's first token, advanced by the walk's stride at
// the end of every token tile without a division; lane offsets below 64
// wrap into the next head(s).
struct TokenWalk {
  int64_t bh0, i0, step_q, step_r, L;
  __host__ __device__ inline void init(int64_t tfirst, int64_t tstep, int64_t L_) {
    L = L_;
    bh0 = tfirst / L;
    i0 = tfirst - bh0 * L;
    step_q = tstep / L;
    step_r = tstep - step_q * L;
  }
  __host__ __device__ inline void advance() {
    bh0 += step_q;
    i0 += step_r;
    if (i0 >= L) {
      i0 -= L;
      ++bh0;
    }
  }
  // (head, position) of the token `off` after the wave's first
  __host__ __device__ inline void at(int off, int64_t& bh, int64_t& i) const {
    bh = bh0;
    i = i0 + off;
    while (i >= L) {  // at most once when L >= 64
      i -= L;
      ++bh;
    }
  }
};

}  // namespace walks
}  // namespace lsh
