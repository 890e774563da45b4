// sort.hip -- stable order of positions by bucket, per (batch, head, round).
//
// Reformer summary (p2.ttnews.xyz), section on LSH attention: positions are
// ordered by bucket, ascending, and by position inside a bucket. Positions of
// a segment are already in increasing order, so a stable counting sort on the
// bucket id alone yields exactly the (bucket, position) order; no pass over
// the position bits is needed.
//
// Phases over tiles of kSortTile positions (one 4-wave workgroup per
// tile; wave w owns the tile's positions 256w .. 256w + 255):
//   count:   counts[seg][tile][b] = how many positions of the tile are in b
//            (LDS atomic adds; the order of the adds does not matter);
//   scan:    per (segment, 256 buckets): rel[seg][tile][b] = the counts of
//            bucket b in earlier tiles, and the bucket's total;
//   starts:  per segment, start[seg][b] = the totals of all buckets < b. The
//            first output slot of the tile's positions in bucket b is
//            start + rel;
//   scatter: each wave first counts its own positions per bucket; a prefix
//            over the waves turns the tile offset into per-wave offsets; then
//            every position gets slot = its wave's offset + (number of earlier
//            positions of the same wave in b), found with wave ballots over
//            the bucket bits (lanes holding equal ids find each other), 64
//            positions at a time in position order.
// Buckets are handled in LDS windows of at most kLdsBins ids, so any
// n_buckets up to 65536 works with a bounded LDS footprint.
//
// Segment form (L <= 16384, n_buckets <= 1024): one launch, one workgroup
// of 16 waves per segment. Wave w owns the positions [w S, (w + 1) S),
// S = L / 16 rounded up to 64-position steps, holds their bucket ids in
// registers, counts them into its own row of a [16][n_buckets] LDS table; the
// table becomes per-wave first slots (an exclusive scan of the bucket totals,
// then a prefix over the waves), and the wave assigns slots 64 positions at a
// time in position order as the scatter above does, into an LDS copy of the
// segment's permutation, which is then stored with coalesced writes
// (scattered 4-byte global stores cost ~2.7 cycles each per CU). Longer
// segments keep the tiled form: ranking costs ~100 vector instructions per
// 64 positions, which the tiled form spreads over every CU.
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

// Exclusive scan of n <= kLdsBins values of src into dst, plus carry (all
// threads of a kSortThreads block call it); returns the sum of the n values.
__device__ uint32_t block_exclusive_scan(const uint32_t* __restrict__ src, uint32_t* dst, int n,
                                         uint32_t carry, uint32_t* wsum) {
  constexpr int kPer = kLdsBins / kSortThreads;
  const int tid = threadIdx.x, lane = tid % kWave, w = tid / kWave;
  uint32_t x[kPer];
  uint32_t sum = 0;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int k = tid * kPer + u;
    x[u] = k < n ? src[k] : 0u;
    sum += x[u];
  }
  uint32_t inc = sum;  // inclusive scan of the thread sums over the wave
#pragma unroll
  for (int off = 1; off < kWave; off <<= 1) {
    const uint32_t y = __shfl_up(inc, off);
    if (lane >= off) inc += y;
  }
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  uint32_t before = carry, total = carry;
  for (int ww = 0; ww < kSortWaves; ++ww) {
    if (ww < w) before += wsum[ww];
    total += wsum[ww];
  }
  uint32_t run = before + inc - sum;
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int k = tid * kPer + u;
    if (k < n) dst[k] = run;
    run += x[u];
  }
  __syncthreads();
  return total - carry;
}

// One block per (segment, 256 buckets), a thread per bucket: the running
// count of the bucket over the tiles replaces each tile's count, all loads of
// a batch of 16 tiles issued before any use, and the bucket's total goes to
// totals[seg][b].
__global__ __launch_bounds__(kSortThreads) void k_sort_scan(uint32_t* __restrict__ counts,
                                                            uint32_t* __restrict__ totals, int nb,
                                                            int tiles, int bblocks) {
  constexpr int kBatch = 16;
  const int64_t seg = blockIdx.x / (unsigned)bblocks;
  const int b = (int)(blockIdx.x - seg * bblocks) * kSortThreads + threadIdx.x;
  if (b >= nb) return;
  uint32_t* c = counts + seg * nb * (int64_t)tiles + b;
  uint32_t run = 0;
  for (int t0 = 0; t0 < tiles; t0 += kBatch) {
    uint32_t x[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) x[u] = t0 + u < tiles ? c[(int64_t)(t0 + u) * nb] : 0u;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (t0 + u < tiles) c[(int64_t)(t0 + u) * nb] = run;
      run += x[u];
    }
  }
  totals[seg * nb + b] = run;
}

// One block per segment: the exclusive scan of the bucket totals gives every
// bucket's first slot, start[seg][b].
__global__ __launch_bounds__(kSortThreads) void k_sort_starts(const uint32_t* __restrict__ totals,
                                                              uint32_t* __restrict__ start,
                                                              int nb) {
  __shared__ uint32_t wsum[kSortWaves];
  const int64_t seg = blockIdx.x;
  uint32_t carry = 0;
  for (int base = 0; base < nb; base += kLdsBins) {
    const int span = min(kLdsBins, nb - base);
    carry += block_exclusive_scan(totals + seg * nb + base, start + seg * nb + base, span, carry,
                                  wsum);
  }
}

__global__ __launch_bounds__(kSortThreads) void k_sort_scatter(
    const uint16_t* __restrict__ buckets, const uint32_t* __restrict__ offsets,
    const uint32_t* __restrict__ start, int32_t* __restrict__ perm, int L, int nb, int tiles,
    int nbits, int64_t nseg) {
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
      uint32_t run = start[seg * nb + base + j] + os[base + j];
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

constexpr int kSegThreads = 1024;
constexpr int kSegWaves = kSegThreads / kWave;
constexpr int kSegMaxBins = 1024;
constexpr int kSegMaxL = 16384;
constexpr int kSegMaxSteps = kSegMaxL / kSegThreads;  // 64-position steps per wave

__global__ __launch_bounds__(kSegThreads) void k_sort_segment(const uint16_t* __restrict__ buckets,
                                                              int32_t* __restrict__ perm, int L,
                                                              int nb, int nbits, int steps) {
  extern __shared__ uint32_t off[];  // [kSegWaves][nb], the wave sums, the permutation
  uint32_t* wsum = off + kSegWaves * nb;
  int32_t* slots = (int32_t*)(wsum + kSegWaves);
  const int64_t seg = blockIdx.x;
  const int t = threadIdx.x, w = t / kWave, lane = t % kWave;
  const uint16_t* bk = buckets + seg * L;
  const int begin = w * steps * kWave;
  for (int j = t; j < kSegWaves * nb; j += kSegThreads) off[j] = 0;
  constexpr uint32_t kNone = 0xFFFFFFFFu;  // no position (past L)
  uint32_t ids[kSegMaxSteps];
#pragma unroll
  for (int k = 0; k < kSegMaxSteps; ++k) {
    const int e = begin + kWave * k + lane;
    ids[k] = k < steps && e < L ? (uint32_t)bk[e] : kNone;
  }
  __syncthreads();
  uint32_t* mine = off + w * nb;
#pragma unroll
  for (int k = 0; k < kSegMaxSteps; ++k)
    if (ids[k] != kNone) atomicAdd(&mine[ids[k]], 1u);
  __syncthreads();
  // thread b: the bucket's total over the waves, its first slot (exclusive
  // scan over the buckets), then each wave's first slot in it
  uint32_t total = 0;
  if (t < nb)
    for (int ww = 0; ww < kSegWaves; ++ww) total += off[ww * nb + t];
  uint32_t inc = total;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == kWave - 1) wsum[w] = inc;
  __syncthreads();
  uint32_t run = inc - total;
  for (int ww = 0; ww < w; ++ww) run += wsum[ww];
  if (t < nb)
    for (int ww = 0; ww < kSegWaves; ++ww) {
      const uint32_t n = off[ww * nb + t];
      off[ww * nb + t] = run;
      run += n;
    }
  __syncthreads();
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int k = 0; k < kSegMaxSteps; ++k) {
    if (k < steps) {  // the same for every wave
      const bool in = ids[k] != kNone;
      const uint64_t peers = match_peers(ids[k], in, nbits);
      if (in) slots[mine[ids[k]] + (uint32_t)__popcll(peers & below)] = begin + kWave * k + lane;
      // all lanes have read the wave's slot above; the group's first lane
      // advances it
      if (in && lane == __builtin_ctzll(peers)) mine[ids[k]] += (uint32_t)__popcll(peers);
    }
  }
  __syncthreads();  // every slot holds its position
  int32_t* pm = perm + seg * L;
  for (int j = t; j < L; j += kSegThreads) pm[j] = slots[j];
}

}  // namespace

hipError_t launch_sort(const Problem& p, const uint16_t* buckets, uint32_t* counts,
                       int32_t* perm, hipStream_t s) {
  int nbits = 0;
  while ((1 << nbits) < p.nb) ++nbits;
  if (p.L <= kSegMaxL && p.nb <= kSegMaxBins) {
    const int steps = (p.L + kSegThreads - 1) / kSegThreads;  // per wave
    const size_t shmem = ((size_t)kSegWaves * p.nb + kSegWaves + p.L) * 4;
    static bool configured[kMaxDevices] = {};
    if (first_on_device(configured))
      (void)hipFuncSetAttribute((const void*)k_sort_segment,
                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                (kSegWaves * kSegMaxBins + kSegWaves + kSegMaxL) * 4);
    hipLaunchKernelGGL(k_sort_segment, dim3((unsigned)p.nseg()), dim3(kSegThreads), shmem, s,
                       buckets, perm, p.L, p.nb, nbits, steps);
    return hipGetLastError();
  }
  // counts: [seg][tiles][nb] tile counts (then their running sums), then the
  // totals and the first slots [seg][nb] of every bucket
  const int tiles = p.sort_tiles();
  uint32_t* totals = counts + p.nseg() * (int64_t)tiles * p.nb;
  uint32_t* start = totals + p.nseg() * (int64_t)p.nb;
  const dim3 grid((unsigned)(tiles * p.nseg()));
  const size_t window = (size_t)(p.nb < kLdsBins ? p.nb : kLdsBins);
  hipLaunchKernelGGL(k_sort_count, grid, dim3(kSortThreads), window * 4, s, buckets, counts, p.L,
                     p.nb, tiles, p.nseg());
  const int bblocks = (p.nb + kSortThreads - 1) / kSortThreads;
  hipLaunchKernelGGL(k_sort_scan, dim3((unsigned)(p.nseg() * bblocks)), dim3(kSortThreads), 0, s,
                     counts, totals, p.nb, tiles, bblocks);
  hipLaunchKernelGGL(k_sort_starts, dim3((unsigned)p.nseg()), dim3(kSortThreads), 0, s, totals,
                     start, p.nb);
  hipLaunchKernelGGL(k_sort_scatter, grid, dim3(kSortThreads), kSortWaves * window * 4, s,
                     buckets, counts, start, perm, p.L, p.nb, tiles, nbits, p.nseg());
  return hipGetLastError();
}

}  // namespace lsh
