// sort.hip -- stable order of positions by bucket, per (batch, head, round).
//
// Reformer summary (p2.ttnews.xyz), section on LSH attention: positions are
// ordered by bucket, ascending, and by position inside a bucket. Positions of
// a segment are already in increasing order, so a stable counting sort on the
// bucket id alone yields exactly the (bucket, position) order; no pass over
// the position bits is needed.
//
// Three phases over tiles of kSortTile positions (one wave per tile):
//   count:   counts[seg][tile][b] = how many positions of the tile are in b;
//   scan:    offsets[seg][tile][b] = sum of all counts of buckets < b plus the
//            counts of bucket b in earlier tiles: the first output slot of the
//            tile's positions in bucket b;
//   scatter: every position gets slot = offset + (number of earlier positions
//            of the same tile in b), computed with wave ballots over the
//            bucket bits (lanes holding equal ids find each other).
// Buckets are handled in LDS windows of at most kLdsBins ids, so any
// n_buckets up to 65536 works with a bounded LDS footprint.
#include "internal.h"

namespace lsh {
namespace {

constexpr int kLdsBins = 8192;

// Mask of active lanes whose key equals this lane's key.
__device__ __forceinline__ uint64_t match_peers(uint32_t key, bool active, int nbits) {
  uint64_t peers = __ballot(active);
  for (int j = 0; j < nbits; ++j) {
    const bool bit = (key >> j) & 1u;
    const uint64_t ones = __ballot(active && bit);
    peers &= bit ? ones : ~ones;
  }
  return peers;
}

__global__ __launch_bounds__(64) void k_sort_count(const uint16_t* __restrict__ buckets,
                                                   uint32_t* __restrict__ counts, int L, int nb,
                                                   int tiles, int nbits) {
  extern __shared__ uint32_t cnt[];
  const int tile = (int)(blockIdx.x % (unsigned)tiles);
  const int64_t seg = blockIdx.x / (unsigned)tiles;
  const int lane = threadIdx.x;
  const uint16_t* bk = buckets + seg * L;
  uint32_t* cs = counts + (seg * tiles + tile) * (int64_t)nb;
  const int begin = tile * kSortTile;
  const int end = min(L, begin + kSortTile);
  const int window = min(nb, kLdsBins);
  for (int base = 0; base < nb; base += window) {
    const int span = min(window, nb - base);
    for (int b = lane; b < span; b += kWave) cnt[b] = 0;
    __syncthreads();
    for (int e0 = begin; e0 < end; e0 += kWave) {
      const int e = e0 + lane;
      const uint32_t b = e < end ? bk[e] : 0u;
      const bool in = e < end && (int)b >= base && (int)b < base + span;
      const uint64_t peers = match_peers(b, in, nbits);
      if (in && lane == __builtin_ctzll(peers)) cnt[b - base] += (uint32_t)__popcll(peers);
    }
    __syncthreads();
    for (int b = lane; b < span; b += kWave) cs[base + b] = cnt[b];
    __syncthreads();
  }
}

// One block per segment. Buckets are taken 1024 at a time, one per thread:
// first the running count over tiles (the tile's offset inside its bucket),
// then a block-wide exclusive scan of the bucket totals gives the bucket's
// first slot, which is added to every tile of the bucket.
__global__ __launch_bounds__(1024) void k_sort_scan(uint32_t* __restrict__ counts, int nb,
                                                    int tiles) {
  __shared__ uint32_t part[1024];
  const int tid = threadIdx.x;
  uint32_t* c = counts + (int64_t)blockIdx.x * nb * tiles;
  uint32_t carry = 0;
  for (int b0 = 0; b0 < nb; b0 += 1024) {
    const int b = b0 + tid;
    uint32_t run = 0;
    if (b < nb) {
      for (int t = 0; t < tiles; ++t) {
        uint32_t* p = c + (int64_t)t * nb + b;
        const uint32_t x = *p;
        *p = run;
        run += x;
      }
    }
    part[tid] = run;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const uint32_t add = tid >= off ? part[tid - off] : 0u;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    const uint32_t base = carry + part[tid] - run;  // exclusive
    if (b < nb)
      for (int t = 0; t < tiles; ++t) c[(int64_t)t * nb + b] += base;
    carry += part[1023];
    __syncthreads();
  }
}

__global__ __launch_bounds__(64) void k_sort_scatter(const uint16_t* __restrict__ buckets,
                                                     const uint32_t* __restrict__ offsets,
                                                     int32_t* __restrict__ perm, int L, int nb,
                                                     int tiles, int nbits) {
  extern __shared__ uint32_t next[];
  const int tile = (int)(blockIdx.x % (unsigned)tiles);
  const int64_t seg = blockIdx.x / (unsigned)tiles;
  const int lane = threadIdx.x;
  const uint16_t* bk = buckets + seg * L;
  const uint32_t* os = offsets + (seg * tiles + tile) * (int64_t)nb;
  int32_t* pm = perm + seg * L;
  const int begin = tile * kSortTile;
  const int end = min(L, begin + kSortTile);
  const uint64_t below = (1ull << lane) - 1ull;
  const int window = min(nb, kLdsBins);
  for (int base = 0; base < nb; base += window) {
    const int span = min(window, nb - base);
    for (int b = lane; b < span; b += kWave) next[b] = os[base + b];
    __syncthreads();
    for (int e0 = begin; e0 < end; e0 += kWave) {
      const int e = e0 + lane;
      const uint32_t b = e < end ? bk[e] : 0u;
      const bool in = e < end && (int)b >= base && (int)b < base + span;
      const uint64_t peers = match_peers(b, in, nbits);
      if (in) {
        const uint32_t slot = next[b - base] + (uint32_t)__popcll(peers & below);
        pm[slot] = e;
      }
      // all lanes have read next[] above; the group's first lane advances it
      if (in && lane == __builtin_ctzll(peers)) next[b - base] += (uint32_t)__popcll(peers);
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_sort(const Problem& p, const uint16_t* buckets, uint32_t* counts,
                       int32_t* perm, hipStream_t s) {
  const int tiles = p.sort_tiles();
  int nbits = 0;
  while ((1 << nbits) < p.nb) ++nbits;
  const dim3 grid((unsigned)(tiles * p.nseg()));
  const size_t lds = (size_t)(p.nb < kLdsBins ? p.nb : kLdsBins) * 4;
  hipLaunchKernelGGL(k_sort_count, grid, dim3(kWave), lds, s, buckets, counts, p.L, p.nb, tiles,
                     nbits);
  hipLaunchKernelGGL(k_sort_scan, dim3((unsigned)p.nseg()), dim3(1024), 0, s, counts, p.nb,
                     tiles);
  hipLaunchKernelGGL(k_sort_scatter, grid, dim3(kWave), lds, s, buckets, counts, perm, p.L,
                     p.nb, tiles, nbits);
  return hipGetLastError();
}

}  // namespace lsh
