// gemm_core.h -- one BM-row x BN-column tile of A B^T on gfx950 matrix cores:
// A [M, K] and B [N, K] bf16 row-major (K contiguous; B is a linear layer's
// weight), fp32 accumulators, v_mfma_f32_16x16x32_bf16.
//
// tile(): a workgroup of WM x WN waves (4 by default), each owning a block of
// BM/WM rows x BN/WN columns. K goes in slabs of SLAB (32 or 64),
// double-buffered in LDS (rows of A and of B, K contiguous, +16-byte pad: the
// 16 lanes of a fragment read distinct bank groups), with the next two slabs
// in flight in two named register sets while the current one is multiplied.
// tile_pp(): 256 x 256 on 8 waves in two groups that take turns at the matrix
// pipe (below).
// Loads are buffer loads through resources in scalar registers, each piece at
// a fixed 32-bit offset (so 256 K * 2 bytes must stay below 2^31), and every
// load and store is unconditional: rows of A past M read row M - 1 (the caller
// does not store them), slabs past the end re-read the last one. (A load or
// store behind a branch makes the compiler drain every load in flight after
// the branch.) Every output element is summed over K in ascending 32-wide
// steps whatever the tile shape or slab, so all shapes give identical results.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;  // threads of the default 2 x 2 wave grid

template <int BM, int BN, int SLAB, int WM = 2, int WN = 2>
struct Lay {
  static constexpr int kThr = 64 * WM * WN;
  static constexpr int kStride = SLAB * 2 + 16;     // bytes per staged row (+16 pad)
  static constexpr int kA = 0;                      // [2][BM] rows of A
  static constexpr int kB = kA + 2 * BM * kStride;  // [2][BN] rows of B
  static constexpr int kBytes = kB + 2 * BN * kStride;
  static constexpr int RT = BM / WM / 16;           // 16-row tiles per wave
  static constexpr int CT = BN / WN / 16;           // 16-column tiles per wave
};

// The lane's outputs: acc[i][ct][u] is row wave_row<BM>(w) + 16i + 4(lane/16) + u,
// column wave_col<BN>(w) + 16ct + lane%16 of the tile.
template <int BM, int WM = 2, int WN = 2>
__device__ __forceinline__ int wave_row(int w) { return (BM / WM) * (w / WN); }
template <int BN, int WN = 2>
__device__ __forceinline__ int wave_col(int w) { return (BN / WN) * (w % WN); }

// A B^T for rows row0 .. row0 + BM - 1 of A and the BN rows of B at brows (K a
// multiple of SLAB). Ends with a barrier: the LDS may be reused at once.
template <int BM, int BN, int SLAB, int WM = 2, int WN = 2>
__device__ __forceinline__ void tile(unsigned char* lds, const uint4* __restrict__ a,
                                     int64_t row0, int64_t M, const uint4* __restrict__ brows,
                                     int K,
                                     floatx4_t (&acc)[Lay<BM, BN, SLAB, WM, WN>::RT][Lay<BM, BN, SLAB, WM, WN>::CT]) {
  using L = Lay<BM, BN, SLAB, WM, WN>;
  constexpr int kThreads = L::kThr;
  constexpr int kP = SLAB / 8;               // 16-byte pieces per staged row
  constexpr int kStride = L::kStride;
  constexpr int kAPer = BM * kP / kThreads;  // 16-byte pieces of the A slab per thread
  constexpr int kBPer = BN * kP / kThreads;  // of the B slab
  static_assert(kAPer >= 1 && kBPer >= 1, "each thread stages a piece of A and of B");
  constexpr int RT = L::RT, CT = L::CT;
  const int t = threadIdx.x;
  const int kseg = K / 8;  // 16-byte pieces per row
  const int nslab = K / SLAB;
  // two slabs in flight in registers (slab j in set j % 2). The loads are
  // buffer loads through two resources held in scalar registers (the tile's
  // rows of A, the BN rows of B), each piece at a fixed 32-bit offset plus the
  // slab's; rows of A past M read row M - 1 (their results are not stored),
  // so no load is conditional.
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const int64_t arows = (M - row0 < BM ? M - row0 : BM);  // rows of A this tile reads
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a + row0 * kseg), (short)0, (int)(arows * K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t bres =
      __builtin_amdgcn_make_buffer_rsrc((void*)brows, (short)0, BN * K * 2, 0x00020000);
  u32x4 ra0[kAPer], rb0[kBPer], ra1[kAPer], rb1[kBPer];
  int aoff[kAPer], boff[kBPer];
#pragma unroll
  for (int j = 0; j < kAPer; ++j) {
    const int r = t / kP + (kThreads / kP) * j;
    aoff[j] = ((r < arows ? r : (int)arows - 1) * kseg + t % kP) * 16;
  }
#pragma unroll
  for (int j = 0; j < kBPer; ++j) boff[j] = ((t / kP + (kThreads / kP) * j) * kseg + t % kP) * 16;
  auto load = [&](u32x4 (&ra)[kAPer], u32x4 (&rb)[kBPer], int s) {
    const int so = s * SLAB * 2;
#pragma unroll
    for (int j = 0; j < kAPer; ++j) ra[j] = __builtin_amdgcn_raw_buffer_load_b128(ares, aoff[j] + so, 0, 0);
#pragma unroll
    for (int j = 0; j < kBPer; ++j) rb[j] = __builtin_amdgcn_raw_buffer_load_b128(bres, boff[j] + so, 0, 0);
  };
  auto store = [&](const u32x4 (&ra)[kAPer], const u32x4 (&rb)[kBPer], int buf) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
      const int r = t / kP + (kThreads / kP) * j, pc = t % kP;
      *(u32x4*)(lds + L::kA + (buf * BM + r) * kStride + pc * 16) = ra[j];
    }
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
      const int c = t / kP + (kThreads / kP) * j, pc = t % kP;
      *(u32x4*)(lds + L::kB + (buf * BN + c) * kStride + pc * 16) = rb[j];
    }
  };

  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const int wr = wave_row<BM, WM, WN>(w), wc = wave_col<BN, WN>(w);
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[i][ct] = floatx4_t{};

  // (raised wave priority while issuing the products: a wave that holds its
  // operands keeps the matrix pipe fed ahead of the other wave's loads)
  auto compute = [&](int buf) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < SLAB / 32; ++ks) {
      bf16x8_t a[RT], b[CT];
#pragma unroll
      for (int i = 0; i < RT; ++i)
        a[i] = *(const bf16x8_t*)(lds + L::kA + (buf * BM + wr + 16 * i + lq) * kStride +
                                  (32 * ks + 8 * g) * 2);
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
        b[ct] = *(const bf16x8_t*)(lds + L::kB + (buf * BN + wc + 16 * ct + lq) * kStride +
                                   (32 * ks + 8 * g) * 2);
#pragma unroll
      for (int i = 0; i < RT; ++i)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
          acc[i][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[ct], acc[i][ct], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
  };

  // (the stores of the clamped slabs past the end land in a buffer no wave
  // reads again)
  const int last = nslab - 1;
  load(ra0, rb0, 0);
  store(ra0, rb0, 0);
  load(ra1, rb1, min(1, last));
  load(ra0, rb0, min(2, last));
  __syncthreads();
  // step s: multiply slab s (LDS buffer s % 2), stage slab s + 1 from its
  // registers, then reuse them for slab s + 3
  for (int s = 0; s < nslab; s += 2) {
    compute(0);
    store(ra1, rb1, 1);
    __syncthreads();
    load(ra1, rb1, min(s + 3, last));
    if (s + 1 < nslab) compute(1);
    store(ra0, rb0, 0);
    __syncthreads();
    load(ra0, rb0, min(s + 4, last));
  }
}

// The same product for BM = BN = 256 on 8 waves (a 4 x 2 wave grid, each wave
// 64 rows x 128 columns, the accumulator layout of tile<256, 256, 32, 4, 2>),
// with the waves in two groups that alternate: waves 0-3 (one per SIMD) load
// the slabs of A, waves 4-7 those of B, and while one group multiplies the
// slab whose operands it holds in registers, the other issues the loads of a
// later slab and reads its operands of the same slab from LDS. Every phase
// ends with a barrier and group 1 runs one phase behind group 0, so each SIMD
// always has one wave issuing products. The slabs go from memory straight
// into LDS (buffer loads with the LDS as destination: no staging registers or
// stores) through a ring of four stages of 256 rows of A then of B, 64 bytes
// per row, loaded three slabs ahead; within each 16-row block the 16-byte
// piece p of row r sits in slot p ^ ((r / 4) % 4), so the 16 lanes of a
// fragment read distinct banks. One load instruction fills a 16-row block
// (1 KB): lane l writes row l / 4, slot l % 4, and so loads piece
// (l % 4) ^ ((l / 16) % 4) of its row. The barriers carry no memory fence (a
// fence would wait for every load in flight): each wave waits for its own part
// of the next slab by vmcnt and for its fragment reads by lgkmcnt before the
// barrier, which the compiler does not do for loads into LDS. K must be a
// multiple of 32. Sums are taken in the same order as tile(): identical
// results.
struct LayPP {
  static constexpr int kThr = 512;
  static constexpr int kHalf = 256 * 64;            // 256 rows of A (or B), one K slab
  static constexpr int kStage = 2 * kHalf;          // [A | B]
  static constexpr int kStages = 4;
  static constexpr int kBytes = kStages * kStage;
  static constexpr int RT = 4, CT = 8;
};

template <int N>
__device__ __forceinline__ void pp_wait_vm() {
  // s_waitcnt vmcnt(N), no wait on the other counters
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x70 | 0xF00);
}

__device__ __forceinline__ void tile_pp(unsigned char* lds, const uint4* __restrict__ a,
                                        int64_t row0, int64_t M, const uint4* __restrict__ brows,
                                        int K, floatx4_t (&acc)[4][8]) {
  typedef __attribute__((address_space(3))) void* lptr_t;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int w = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool gb = w >= 4;  // group 1 stages B
  const int kseg = K / 8;
  const int nslab = K / 32;
  const int last = nslab - 1;
  const int64_t arows = (M - row0 < 256 ? M - row0 : 256);
  const __amdgpu_buffer_rsrc_t ares = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(a + row0 * kseg), (short)0, (int)(arows * K * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t bres =
      __builtin_amdgcn_make_buffer_rsrc((void*)brows, (short)0, 256 * K * 2, 0x00020000);
  const __amdgpu_buffer_rsrc_t res = gb ? bres : ares;
  const int nrows = gb ? 256 : (int)arows;
  // wave w % 4 of the group loads the 16-row blocks 4 (w % 4) + j of its half
  // (one 1 KB block per load: lane l writes row l / 4 of the block, slot l % 4,
  // and so fetches piece (l % 4) ^ ((l / 16) % 4) of that row)
  const int wg = w & 3;
  const int lpiece = (lane & 3) ^ ((lane >> 4) & 3);
  int off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int r = 16 * (4 * wg + j) + (lane >> 2);
    off[j] = ((r < nrows ? r : nrows - 1) * kseg + lpiece) * 16;
  }
  unsigned char* const hbase = lds + (gb ? LayPP::kHalf : 0) + 4 * wg * 1024;
  auto dma = [&](int s) {
    unsigned char* dst = hbase + (s & 3) * LayPP::kStage;
    const int so = (s < last ? s : last) * 64;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (lptr_t)(dst + j * 1024), 16, off[j], so, 0,
                                               0);
  };
  const int g = lane >> 4, lq = lane & 15;
  const int wr = 64 * (w / 2), wc = 128 * (w % 2);
  const int slot = 16 * (g ^ (lq >> 2));
  const int arel = (wr + lq) * 64 + slot;
  const int brel = LayPP::kHalf + (wc + lq) * 64 + slot;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) acc[i][ct] = floatx4_t{};
  bf16x8_t fa[4], fb[8];
  auto read = [&](int s) {
    const unsigned char* st = lds + (s & 3) * LayPP::kStage;
#pragma unroll
    for (int i = 0; i < 4; ++i) fa[i] = *(const bf16x8_t*)(st + arel + i * 1024);
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) fb[ct] = *(const bf16x8_t*)(st + brel + ct * 1024);
  };
  auto compute = [&]() {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
        acc[i][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[ct], acc[i][ct], 0, 0, 0);
  };
  // barriers without a memory fence: the waits are explicit (the loads into
  // LDS by vmcnt, the fragment reads by lgkmcnt), so the slab loads stay in
  // flight across them
  auto bar = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };
  auto lgkm0 = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
  };
  auto vm8 = [&]() {
    __builtin_amdgcn_sched_barrier(0);
    pp_wait_vm<8>();
    __builtin_amdgcn_sched_barrier(0);
  };

  dma(0);
  dma(1);
  dma(2);
  vm8();  // slab 0 of this wave is in LDS
  bar();
  if (gb) bar();  // group 1 runs one phase behind
  for (int s = 0; s < nslab; ++s) {
    // memory phase: slab s + 3 on its way, slab s + 1 (this wave's part) in
    // LDS, then this wave's operands of slab s
    dma(s + 3);
    vm8();
    read(s);
    lgkm0();
    bar();
    compute();
    bar();
  }
  if (!gb) bar();
  // the loads of the clamped slabs past the end: drain them before the
  // caller reuses the LDS
  __builtin_amdgcn_sched_barrier(0);
  pp_wait_vm<0>();
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
}

}  // namespace gemm
}  // namespace lsh
