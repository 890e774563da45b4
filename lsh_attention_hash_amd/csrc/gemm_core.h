// gemm_core.h -- one BM-row x BN-column tile of A B^T on gfx950 matrix cores:
// A [M, K] and B [N, K] bf16 row-major (K contiguous; B is a linear layer's
// weight), fp32 accumulators, v_mfma_f32_16x16x32_bf16.
//
// A workgroup of WM x WN waves (4 by default), each owning a block of BM/WM
// rows x BN/WN columns. K goes
// in slabs of SLAB (32 or 64), double-buffered in LDS (rows of A and of B, K
// contiguous, +16-byte pad: the 16 lanes of a fragment read distinct bank
// groups), with the next two slabs in flight in two named register sets while
// the current one is multiplied. Loads are branch-free: rows of A past M read
// row M - 1 (the caller does not store them). Every output element is summed
// over K in ascending 32-wide steps whatever the tile shape or slab, so the
// shapes give identical results.
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
  // two slabs in flight in registers (slab j in set j % 2); rows past M
  // read row M - 1 (their results are not stored), so no load is conditional
  uint4 ra0[kAPer], rb0[kBPer], ra1[kAPer], rb1[kBPer];
  int64_t arow[kAPer];
#pragma unroll
  for (int j = 0; j < kAPer; ++j) {
    const int64_t row = row0 + t / kP + (kThreads / kP) * j;
    arow[j] = (row < M ? row : M - 1) * kseg + t % kP;
  }
  const uint4* bbase = brows + (int64_t)(t / kP) * kseg + t % kP;
  auto load = [&](uint4 (&ra)[kAPer], uint4 (&rb)[kBPer], int s) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) ra[j] = a[arow[j] + s * kP];
#pragma unroll
    for (int j = 0; j < kBPer; ++j) rb[j] = bbase[(int64_t)(kThreads / kP) * j * kseg + s * kP];
  };
  // (each piece passes through a register-only asm statement, so the copy
  // cannot become a memcpy from a stack copy of the registers)
  auto store = [&](const uint4 (&ra)[kAPer], const uint4 (&rb)[kBPer], int buf) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
      const int r = t / kP + (kThreads / kP) * j, pc = t % kP;
      uint4 q = ra[j];
      asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
      *(uint4*)(lds + L::kA + (buf * BM + r) * kStride + pc * 16) = q;
    }
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
      const int c = t / kP + (kThreads / kP) * j, pc = t % kP;
      uint4 q = rb[j];
      asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
      *(uint4*)(lds + L::kB + (buf * BN + c) * kStride + pc * 16) = q;
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

  load(ra0, rb0, 0);
  store(ra0, rb0, 0);
  if (1 < nslab) load(ra1, rb1, 1);
  if (2 < nslab) load(ra0, rb0, 2);
  __syncthreads();
  // step s: multiply slab s (LDS buffer s % 2), stage slab s + 1 from its
  // registers, then reuse them for slab s + 3
  for (int s = 0; s < nslab; s += 2) {
    compute(0);
    if (s + 1 < nslab) store(ra1, rb1, 1);
    __syncthreads();
    if (s + 3 < nslab) load(ra1, rb1, s + 3);
    if (s + 1 < nslab) {
      compute(1);
      if (s + 2 < nslab) store(ra0, rb0, 0);
      __syncthreads();
      if (s + 4 < nslab) load(ra0, rb0, s + 4);
    }
  }
}

}  // namespace gemm
}  // namespace lsh
