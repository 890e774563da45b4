// gemm_core.h -- one 128-row x BN-column tile of A B^T on gfx950 matrix cores:
// A [M, K] and B [N, K] bf16 row-major (K contiguous; B is a linear layer's
// weight), fp32 accumulators, v_mfma_f32_16x16x32_bf16.
//
// A workgroup of 4 waves as 2 x 2 blocks of 64 rows x BN/2 columns. K goes in
// slabs of 64, double-buffered in LDS (rows of A and of B, K contiguous,
// +16-byte pad: the 16 lanes of a fragment read distinct bank groups), with
// the next two slabs in flight in two named register sets while the current
// one is multiplied. Loads are branch-free: rows of A past M read row M - 1
// (the caller does not store them).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lsh {
namespace gemm {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kRows = 128;               // rows of A per tile
constexpr int kSlab = 64;                // K per LDS slab
constexpr int kStride = kSlab * 2 + 16;  // bytes per staged row (+16 pad)

template <int BN>
struct Lay {
  static constexpr int kA = 0;                          // [2][kRows] rows of A
  static constexpr int kB = kA + 2 * kRows * kStride;   // [2][BN] rows of B
  static constexpr int kBytes = kB + 2 * BN * kStride;
  static constexpr int RT = 4;                          // 16-row tiles per wave
  static constexpr int CT = BN / 32;                    // 16-column tiles per wave
};

// The lane's outputs: acc[i][ct][u] is row wave_row(w) + 16i + 4(lane/16) + u,
// column wave_col<BN>(w) + 16ct + lane%16 of the tile.
__device__ __forceinline__ int wave_row(int w) { return 64 * (w >> 1); }
template <int BN>
__device__ __forceinline__ int wave_col(int w) { return (BN / 2) * (w & 1); }

// A B^T for rows row0 .. row0 + 127 of A and the BN rows of B at brows (K a
// multiple of 64). Ends with a barrier: the LDS may be reused at once.
template <int BN>
__device__ __forceinline__ void tile(unsigned char* lds, const uint4* __restrict__ a,
                                     int64_t row0, int64_t M, const uint4* __restrict__ brows,
                                     int K,
                                     floatx4_t (&acc)[Lay<BN>::RT][Lay<BN>::CT]) {
  using L = Lay<BN>;
  constexpr int kAPer = kRows * 8 / kThreads;  // 16-byte pieces of the A slab per thread
  constexpr int kBPer = BN * 8 / kThreads;     // of the B slab
  constexpr int RT = L::RT, CT = L::CT;
  const int t = threadIdx.x;
  const int kseg = K / 8;  // 16-byte pieces per row
  const int nslab = K / kSlab;
  // two slabs in flight in registers (slab j in set j % 2); rows past M
  // read row M - 1 (their results are not stored), so no load is conditional
  uint4 ra0[kAPer], rb0[kBPer], ra1[kAPer], rb1[kBPer];
  int64_t arow[kAPer];
#pragma unroll
  for (int j = 0; j < kAPer; ++j) {
    const int64_t row = row0 + t / 8 + (kThreads / 8) * j;
    arow[j] = (row < M ? row : M - 1) * kseg + t % 8;
  }
  const uint4* bbase = brows + (int64_t)(t / 8) * kseg + t % 8;
  auto load = [&](uint4 (&ra)[kAPer], uint4 (&rb)[kBPer], int s) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) ra[j] = a[arow[j] + s * 8];
#pragma unroll
    for (int j = 0; j < kBPer; ++j) rb[j] = bbase[(int64_t)(kThreads / 8) * j * kseg + s * 8];
  };
  // (each piece passes through a register-only asm statement, so the copy
  // cannot become a memcpy from a stack copy of the registers)
  auto store = [&](const uint4 (&ra)[kAPer], const uint4 (&rb)[kBPer], int buf) {
#pragma unroll
    for (int j = 0; j < kAPer; ++j) {
      const int r = t / 8 + (kThreads / 8) * j, pc = t % 8;
      uint4 q = ra[j];
      asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
      *(uint4*)(lds + L::kA + (buf * kRows + r) * kStride + pc * 16) = q;
    }
#pragma unroll
    for (int j = 0; j < kBPer; ++j) {
      const int c = t / 8 + (kThreads / 8) * j, pc = t % 8;
      uint4 q = rb[j];
      asm volatile("" : "+v"(q.x), "+v"(q.y), "+v"(q.z), "+v"(q.w));
      *(uint4*)(lds + L::kB + (buf * BN + c) * kStride + pc * 16) = q;
    }
  };

  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const int wr = wave_row(w), wc = wave_col<BN>(w);
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) acc[i][ct] = floatx4_t{};

  auto compute = [&](int buf) {
#pragma unroll
    for (int ks = 0; ks < kSlab / 32; ++ks) {
      bf16x8_t a[RT], b[CT];
#pragma unroll
      for (int i = 0; i < RT; ++i)
        a[i] = *(const bf16x8_t*)(lds + L::kA + (buf * kRows + wr + 16 * i + lq) * kStride +
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
