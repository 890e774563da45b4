// sort.hip -- stable order of positions by bucket, per (batch, head, round).
//
// Reformer summary (p2.ttnews.xyz), section on LSH attention: positions are
// ordered by bucket, ascending, and by position inside a bucket. Positions of
// a segment are already in increasing order, so a stable counting sort on the
// bucket id alone yields exactly the (bucket, position) order; no pass over
// the position bits is needed.
//
// Three phases over tiles of kSortTile positions (one 4-wave workgroup per
// tile; wave w owns the tile's positions 256w .. 256w + 255):
//   count:   counts[seg][tile][b] = how many positions of the tile are in b
//            (LDS atomic adds; the order of the adds does not matter);
//   scan:    offsets[seg][tile][b] = sum of all counts of buckets < b plus the
//            counts of bucket b in earlier tiles: the first output slot of the
//            tile's positions in bucket b;
//   scatter: each wave first counts its own positions per bucket; a prefix
//            over the waves turns the tile offset into per-wave offsets; then
//            every position gets slot = its wave's offset + (number of earlier
//            positions of the same wave in b), found with wave ballots over
//            the bucket bits (lanes holding equal ids find each other), 64
//            positions at a time in position order.
// Buckets are handled in LDS windows of at most kLdsBins ids, so any
// n_buckets up to 65536 works with a bounded LDS footprint.
#include "internal.h"
#include "walks.h"

namespace lsh {
namespace {

constexpr int kLdsBins = 2048;
constexpr int kSortThreads = 256;
constexpr int kSortWaves = kSortThreads / kWave;
constexpr int kPerThread = kSortTile / kSortThreads;  // positions per thread
static_assert(kPerThread * kSortThreads == kSortTile, "tile covered by the workgroup");

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

// Workgroups are dealt to the 8 XCDs round-robin (walks.h: block b takes a
// tile of a segment on b's XCD when the segments split evenly).
__device__ __forceinline__ void block_tile(int tiles, int64_t nseg, int64_t& seg, int& tile) {
  walks::sort_block_tile(blockIdx.x, tiles, nseg, seg, tile);
}

// Thread (w, lane) takes positions begin + 256w + 64k + lane, k = 0..3: in
// position order per wave, one coalesced 128-byte read per wave and k.
__device__ __forceinline__ void load_tile(const uint16_t* bk, int begin, int end, uint32_t* b,
                                          int* e) {
  const int w = threadIdx.x / kWave, lane = threadIdx.x % kWave;
#pragma unroll
  for (int k = 0; k < kPerThread; ++k) {
    e[k] = begin + kWave * (kPerThread * w + k) + lane;
    b[k] = e[k] < end ? bk[e[k]] : 0u;
  }
}

__global__ __launch_bounds__(kSortThreads) void k_sort_count(const uint16_t* __restrict__ buckets,
                                                             uint32_t* __restrict__ counts, int L,
                                                             int nb, int tiles, int64_t nseg) {
  extern __shared__ uint32_t cnt[];
  int64_t seg;
  int tile;
  block_tile(tiles, nseg, seg, tile);
  const int tid = threadIdx.x;
  uint32_t* cs = counts + (seg * tiles + tile) * (int64_t)nb;
  const int begin = tile * kSortTile;
  const int end = min(L, begin + kSortTile);
  uint32_t b[kPerThread];
  int e[kPerThread];
  load_tile(buckets + seg * L, begin, end, b, e);
  const int window = min(nb, kLdsBins);
  for (int base = 0; base < nb; base += window) {
    const int span = min(window, nb - base);
    for (int j = tid; j < span; j += kSortThreads) cnt[j] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
      if (e[k] < end && (int)b[k] >= base && (int)b[k] < base + span) atomicAdd(&cnt[b[k] - base], 1u);
    __syncthreads();
    for (int j = tid; j < span; j += kSortThreads) cs[base + j] = cnt[j];
    __syncthreads();
  }
}

// One block per segment. Buckets are taken 1024 at a time, one per thread:
// first the bucket's total over the tiles, then a block-wide exclusive scan
// of the totals gives the bucket's first slot, and a second pass over the
// tiles replaces every count with the running slot. Counts are read 16 tiles
// at a time, all loads of a batch issued before any use.
__global__ __launch_bounds__(1024) void k_sort_scan(uint32_t* __restrict__ counts, int nb,
                                                    int tiles) {
  constexpr int kBatch = 16;
  __shared__ uint32_t part[1024];
  const int tid = threadIdx.x;
  uint32_t* c = counts + (int64_t)blockIdx.x * nb * tiles;
  uint32_t carry = 0;
  for (int b0 = 0; b0 < nb; b0 += 1024) {
    const int b = b0 + tid;
    uint32_t total = 0;
    if (b < nb) {
      for (int t0 = 0; t0 < tiles; t0 += kBatch) {
        uint32_t x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) x[u] = t0 + u < tiles ? c[(int64_t)(t0 + u) * nb + b] : 0u;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) total += x[u];
      }
    }
    part[tid] = total;
    __syncthreads();
    for (int off = 1; off < 1024; off <<= 1) {
      const uint32_t add = tid >= off ? part[tid - off] : 0u;
      __syncthreads();
      part[tid] += add;
      __syncthreads();
    }
    uint32_t run = carry + part[tid] - total;  // exclusive
    if (b < nb) {
      for (int t0 = 0; t0 < tiles; t0 += kBatch) {
        uint32_t x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) x[u] = t0 + u < tiles ? c[(int64_t)(t0 + u) * nb + b] : 0u;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (t0 + u < tiles) c[(int64_t)(t0 + u) * nb + b] = run;
          run += x[u];
        }
      }
    }
    carry += part[1023];
    __syncthreads();
  }
}

__global__ __launch_bounds__(kSortThreads) void k_sort_scatter(
    const uint16_t* __restrict__ buckets, const uint32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int L, int nb, int tiles, int nbits, int64_t nseg) {
  extern __shared__ uint32_t next[];  // [wave][window]
  int64_t seg;
  int tile;
  block_tile(tiles, nseg, seg, tile);
  const int tid = threadIdx.x;
  const int w = tid / kWave, lane = tid % kWave;
  const uint32_t* os = offsets + (seg * tiles + tile) * (int64_t)nb;
  int32_t* pm = perm + seg * L;
  const int begin = tile * kSortTile;
  const int end = min(L, begin + kSortTile);
  const uint64_t below = (1ull << lane) - 1ull;
  uint32_t b[kPerThread];
  int e[kPerThread];
  load_tile(buckets + seg * L, begin, end, b, e);
  const int window = min(nb, kLdsBins);
  for (int base = 0; base < nb; base += window) {
    const int span = min(window, nb - base);
    uint32_t* mine = next + w * span;
    for (int j = tid; j < kSortWaves * span; j += kSortThreads) next[j] = 0;
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPerThread; ++k)
      if (e[k] < end && (int)b[k] >= base && (int)b[k] < base + span)
        atomicAdd(&mine[b[k] - base], 1u);
    __syncthreads();
    for (int j = tid; j < span; j += kSortThreads) {
      uint32_t run = os[base + j];
#pragma unroll
      for (int ww = 0; ww < kSortWaves; ++ww) {
        const uint32_t n = next[ww * span + j];
        next[ww * span + j] = run;
        run += n;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kPerThread; ++k) {
      const bool in = e[k] < end && (int)b[k] >= base && (int)b[k] < base + span;
      const uint64_t peers = match_peers(b[k], in, nbits);
      if (in) {
        const uint32_t slot = mine[b[k] - base] + (uint32_t)__popcll(peers & below);
        pm[slot] = e[k];
      }
      // all lanes have read the wave's counter above; the group's first lane
      // advances it
      if (in && lane == __builtin_ctzll(peers)) mine[b[k] - base] += (uint32_t)__popcll(peers);
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
  const size_t window = (size_t)(p.nb < kLdsBins ? p.nb : kLdsBins);
  hipLaunchKernelGGL(k_sort_count, grid, dim3(kSortThreads), window * 4, s, buckets, counts, p.L,
                     p.nb, tiles, p.nseg());
  hipLaunchKernelGGL(k_sort_scan, dim3((unsigned)p.nseg()), dim3(1024), 0, s, counts, p.nb,
                     tiles);
  hipLaunchKernelGGL(k_sort_scatter, grid, dim3(kSortThreads), kSortWaves * window * 4, s,
                     buckets, counts, perm, p.L, p.nb, tiles, nbits, p.nseg());
  return hipGetLastError();
}

}  // namespace lsh
