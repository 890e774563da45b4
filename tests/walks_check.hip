// Host-side check of the grid walks the chunked kernels run
// (lsh_attention_hash_amd/csrc/walks.h): the same functions, over whole grids
// of many shapes, with every index checked against its bound and every unit
// of work required to be visited exactly once. Runs on the CPU (no HIP call).
// Built and run by tests/test_walks.py; prints "walks ok" and exits 0, or
// prints the first failure and exits 1.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "walks.h"

using namespace lsh::walks;

static int fail(const char* what, long long a, long long b, long long c) {
  std::printf("FAIL %s (%lld, %lld, %lld)\n", what, a, b, c);
  return 1;
}

// attention / backward range walk: every (segment, chunk) once
static int check_ranges(int nchunks, int64_t nseg, int R, int max_per, int64_t resident) {
  const RangeShape sh = range_shape(nchunks, nseg, R, max_per, resident);
  if (sh.per < 1 || sh.ranges < 1 || sh.group_segs < 1 || sh.group_segs > nseg ||
      sh.blocks != nseg * sh.ranges || (int64_t)sh.per * sh.ranges < nchunks)
    return fail("range shape", nchunks, nseg, R);
  std::vector<unsigned char> seen((size_t)(nseg * nchunks), 0);
  for (int64_t b = 0; b < sh.blocks; ++b) {
    int64_t seg;
    int range;
    range_block((unsigned)b, sh.group_segs, sh.ranges, (int)nseg, seg, range);
    if (seg < 0 || seg >= nseg || range < 0 || range >= sh.ranges)
      return fail("range block out of bounds", b, seg, range);
    const int c0 = range * sh.per;
    const int c1 = c0 + sh.per < nchunks ? c0 + sh.per : nchunks;
    for (int c = c0; c < c1; ++c)
      if (seen[(size_t)(seg * nchunks + c)]++) return fail("chunk visited twice", seg, c, b);
  }
  for (size_t k = 0; k < seen.size(); ++k)
    if (seen[k] != 1) return fail("chunk not visited", (long long)(k / nchunks), (long long)(k % nchunks), nchunks);
  return 0;
}

// sort: every (segment, tile) once
static int check_sort(int tiles, int64_t nseg) {
  std::vector<unsigned char> seen((size_t)(tiles * nseg), 0);
  for (int64_t b = 0; b < tiles * nseg; ++b) {
    int64_t seg;
    int tile;
    sort_block_tile((unsigned)b, tiles, nseg, seg, tile);
    if (seg < 0 || seg >= nseg || tile < 0 || tile >= tiles)
      return fail("sort block out of bounds", b, seg, tile);
    if (seen[(size_t)(seg * tiles + tile)]++) return fail("sort tile twice", seg, tile, b);
    // the XCD-grouped order keeps all tiles of a segment on the block's XCD
    if (nseg % kXcds == 0 && seg % kXcds != b % kXcds) return fail("sort XCD", b, seg, tile);
  }
  return 0;
}

// hash: every (round, token-head) once; the incremental (head, position)
// equals the division; every row index in range. `waves` waves of 64 tokens
// per workgroup (the kernel's token tile: 8), lanes as offsets 0..63 of a wave.
static int check_hash(int64_t BH, int64_t L, int R, int n_cu, int per_cu, int waves) {
  const int kTokWave = 64, kTokWG = waves * kTokWave;
  const int64_t N = BH * L;
  const int n_tok_tiles = (int)((N + kTokWG - 1) / kTokWG);
  const int64_t grid = hash_grid(n_cu, per_cu, R, n_tok_tiles);
  if (grid % (8 * R) != 0 || grid < 8 * R) return fail("hash grid", grid, R, n_tok_tiles);
  const int ngrp = (int)(grid / R);
  std::vector<unsigned char> seen((size_t)(N * R), 0);
  std::vector<unsigned char> block_rg((size_t)(R * ngrp), 0);
  for (int64_t b = 0; b < grid; ++b) {
    int r, grp;
    hash_block((unsigned)b, R, r, grp);
    if (r < 0 || r >= R || grp < 0 || grp >= ngrp) return fail("hash block", b, r, grp);
    if (block_rg[(size_t)(r * ngrp + grp)]++) return fail("hash (round, group) twice", b, r, grp);
    for (int w = 0; w < waves; ++w) {
      TokenWalk tw;
      tw.init((int64_t)grp * kTokWG + w * kTokWave, (int64_t)ngrp * kTokWG, L);
      for (int j = grp; j < n_tok_tiles; j += ngrp) {
        const int64_t tok0 = (int64_t)j * kTokWG + w * kTokWave;
        for (int off = 0; off < kTokWave; ++off) {
          const int64_t n = tok0 + off;
          if (n >= N) continue;  // past the last token-head: not written
          int64_t bh, i;
          tw.at(off, bh, i);
          if (bh != n / L || i != n % L) return fail("hash walk (head, position)", n, bh, i);
          const int64_t row = (bh * R + r) * L + i;
          if (row < 0 || row >= N * R) return fail("hash row", row, bh, i);
          if (seen[(size_t)row]++) return fail("hash row twice", row, r, n);
        }
        tw.advance();
      }
    }
  }
  for (size_t k = 0; k < seen.size(); ++k)
    if (seen[k] != 1) return fail("hash row not visited", (long long)k, R, L);
  return 0;
}

int main() {
  const int nchunks[] = {1, 2, 3, 15, 16, 17, 37, 64, 192, 512, 1024, 2048};
  const int64_t bhs[] = {1, 2, 3, 8, 32, 64};
  for (int nc : nchunks)
    for (int64_t bh : bhs)
      for (int R = 1; R <= 8; ++R)
        for (int64_t resident : {64, 256, 512})
          if (check_ranges(nc, bh * R, R, 16, resident)) return 1;
  for (int tiles : {1, 2, 3, 16, 37, 64, 128})
    for (int64_t nseg : {1, 2, 7, 8, 16, 24, 32, 64, 256})
      if (check_sort(tiles, nseg)) return 1;
  const int64_t Ls[] = {64, 128, 192, 1024, 2368, 4096, 12288};
  for (int64_t L : Ls)
    for (int64_t bh : {1, 2, 3, 8})
      for (int R : {1, 2, 3, 4, 5, 8})
        for (int n_cu : {1, 8, 80, 256})
          for (int per_cu : {1, 2})
            for (int waves : {8, 4})
              if (check_hash(bh, L, R, n_cu, per_cu, waves)) return 1;
  // the bench's largest walks, in full
  for (int waves : {8, 4})
    if (check_hash(8, 65536, 4, 256, 1, waves) || check_hash(64, 12288, 8, 256, 2, waves) ||
        check_hash(16, 32768, 8, 256, 1, waves) || check_hash(3, 1000, 3, 80, 1, waves))
      return 1;
  if (check_ranges(1024, 32, 4, 16, 512) || check_ranges(192, 512, 8, 16, 512) ||
      check_ranges(512, 128, 8, 16, 256))
    return 1;
  std::printf("walks ok\n");
  return 0;
}
