// hash_mfma.hip -- random-rotation bucket ids on gfx950 matrix cores, with an
// exactness certificate.
//
// The bucket of x in round r is the index of the largest entry of
// [x R_r; -x R_r] (Reformer summary, p2.ttnews.xyz, section on LSH), i.e. the
// column k with the largest |p_k|, p = x R_r, shifted by n_buckets/2 when
// p_k < 0. The decision must equal the one made on the exact projection
// (ties aside), so the bulk projection runs in fp16 on the matrix cores and
// every decision is either certified or redone exactly:
//
//  1. prep: R_r is rounded to fp16 (clamped to +-65504, |R| < 2^-14 flushed to
//     0) and stored transposed [r][k][d] with zero columns up to a multiple of
//     32; per round the kernel records upper bounds of max_k |Rh_k|,
//     max_k |R_k - Rh_k| and max_k |R_k| (2-norms over d, computed in fp64).
//     A transposed fp32 copy [r][k][d] serves the exact re-scoring.
//  2. main: x (bf16) is rounded to fp16 the same way (once per forward, in a
//     streaming pre-pass that also records |x16| and |x - x16| per row);
//     v_mfma_f32_32x32x16_f16
//     gives p~ = x16 . Rh_k with exact products and fp32 sums. For every
//     column the kernel forms a key (bits of |p~| with the low ib mantissa bits
//     replaced by k) and keeps the two largest keys per row (max3 / med3).
//     With E = (gamma |Rh|max + |lo|max) |x16| + |R|max |x - x16| bounding
//     | |p~_k| - |p_k| | for every k (Cauchy-Schwarz on each correction term,
//     gamma = (d + 2) 2^-23 for the fp32 accumulation in any order) and S the
//     key truncation (2^(ib-22) of the top value):
//       top1 - top2 > 2 (E + S): the winner is certain; its sign comes from an
//         fp32 recomputation of p~_k1 (|p| > E, so the sign is right);
//       else the row is queued for a rescan, which recomputes the same
//         projections keeping the three largest keys:
//         top1 - top3 > 2 (E + S): only k1, k2 can win -> queue A;
//         else -> queue B (all columns).
//  3. fallback: queue A entries re-score the two candidates, queue B entries
//     every column, in fp64 with t = 0..d-1 in order: the products of a bf16
//     input and an fp32 rotation are exact in fp64, so these sums are the
//     correctly ordered fp64 projections, and the winner follows the rule of
//     the definition (largest entry, lowest index on ties).
#include <float.h>
#include <limits.h>

#include <type_traits>

#include "dtype.h"
#include "hash_x16.h"
#include "internal.h"
#include "walks.h"

namespace lsh {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;     // 8 waves, two per SIMD: one's MFMAs cover the other's waits
constexpr int kTokWave = 64;      // 2 sets of 32 tokens per wave
constexpr int kTokWG = kThreads / 64 * kTokWave;
constexpr int kRotLoads = 8;      // rotation loads per thread in flight (8 x 16 B x 512 = 64 KB)
using hx::f16_round;
using hx::kF16Max;
using hx::kF16MinNormal;

// upper bound of a non-negative double as float
__device__ __forceinline__ float up_f32(double x) { return (float)(x * (1.0 + 1e-6)) + 1e-30f; }

// Rotation preparation, one block of 256 threads per (round, 32-column
// tile) `tb`: 8 groups of 32 threads read R row by row (coalesced over
// columns), the tile is transposed in LDS and written out as rows of d; the
// tile's maxima of |Rh_k|, |R_k - Rh_k| and |R_k| go to part[r][kt] (the
// projection takes the maximum over the round's tiles).
constexpr int kPrepMaxD = 128;
__device__ __forceinline__ void prep_tile(int tb, const float* __restrict__ rot,
                                          _Float16* __restrict__ rh, float* __restrict__ rt,
                                          float4* __restrict__ part, int d, int half,
                                          int half_pad) {
  __shared__ __align__(16) _Float16 th[32][kPrepMaxD + 8];
  __shared__ __align__(16) float tx[32][kPrepMaxD + 4];
  __shared__ double red[3][8][33];
  const int ntiles = half_pad / 32;
  const int kt = tb % ntiles;
  const int r = tb / ntiles;
  const int col = threadIdx.x & 31, grp = threadIdx.x >> 5;
  const int k = kt * 32 + col;
  // every load issued before the first use
  float xs[kPrepMaxD / 8];
#pragma unroll
  for (int i = 0; i < kPrepMaxD / 8; ++i) {
    const int u = grp + 8 * i;
    xs[i] = u < d && k < half ? rot[((int64_t)r * d + u) * half + k] : 0.f;
  }
  double sh = 0.0, slo = 0.0, sr = 0.0;
#pragma unroll
  for (int i = 0; i < kPrepMaxD / 8; ++i) {
    const int u = grp + 8 * i;
    if (u < d) {
      const float x = xs[i];
      const float h = f16_round(x);
      th[col][u] = (_Float16)h;
      tx[col][u] = x;
      const double hd = h, xd = x;
      sh += hd * hd;
      slo += (xd - hd) * (xd - hd);
      sr += xd * xd;
    }
  }
  red[0][grp][col] = sh;
  red[1][grp][col] = slo;
  red[2][grp][col] = sr;
  __syncthreads();
  const int pieces_h = d / 8, pieces_x = d / 4;
  for (int idx = threadIdx.x; idx < 32 * pieces_h; idx += 256) {
    const int row = idx / pieces_h, c = idx % pieces_h;
    *(uint4*)(rh + ((int64_t)r * half_pad + kt * 32 + row) * d + c * 8) = *(const uint4*)&th[row][c * 8];
  }
  for (int idx = threadIdx.x; idx < 32 * pieces_x; idx += 256) {
    const int row = idx / pieces_x, c = idx % pieces_x;
    if (kt * 32 + row < half)
      *(uint4*)(rt + ((int64_t)r * half + kt * 32 + row) * d + c * 4) = *(const uint4*)&tx[row][c * 4];
  }
  if (grp == 0) {
    double a = 0.0, b = 0.0, c = 0.0;
    for (int g2 = 0; g2 < 8; ++g2) {
      a += red[0][g2][col];
      b += red[1][g2][col];
      c += red[2][g2][col];
    }
    float fa = up_f32(sqrt(a)), fb = up_f32(sqrt(b)), fc = up_f32(sqrt(c));
    for (int off = 16; off > 0; off >>= 1) {
      fa = fmaxf(fa, __shfl_xor(fa, off));
      fb = fmaxf(fb, __shfl_xor(fb, off));
      fc = fmaxf(fc, __shfl_xor(fc, off));
    }
    if (col == 0) part[r * ntiles + kt] = make_float4(fa, fb, fc, 0.f);
  }
}

// Keep the three largest of (t1 >= t2 >= t3) and key. Keys have a clear sign
// bit and finite magnitude bits, so as floats they order exactly like their
// bit patterns: the max is an unsigned integer max (no NaN canonicalisation
// on the way), and v_med3_f32 returns one of its inputs; keys below 2^-126
// (rows whose projections are all ~0) may be flushed by the med3, and such
// rows are never certified (their top value is ~0).
__device__ __forceinline__ void top3(uint32_t& t1, uint32_t& t2, uint32_t& t3, uint32_t key) {
  const uint32_t n1 = t1 > key ? t1 : key;
  const float n2 = __builtin_amdgcn_fmed3f(__uint_as_float(t1), __uint_as_float(t2),
                                           __uint_as_float(key));
  const float n3 = __builtin_amdgcn_fmed3f(__uint_as_float(t2), __uint_as_float(t3),
                                           __uint_as_float(key));
  t1 = n1;
  t2 = __float_as_uint(n2);
  t3 = __float_as_uint(n3);
}

// Per row, once per forward for every round: the upper bounds of |x16| and
// |x - x16| that the certificate needs (x16: the fp16 row the projection
// converts in registers, hx::x16_pair), and the squared norm of the bf16 row
// (fp32), which the attention turns into its key scale; block `blk` of
// `nblk`. 4 consecutive lanes share a row (D/32 16-byte pieces each), two
// rows per lane group in flight. With kX16 = false only the squared norms
// are produced.
constexpr int kNormLanes = 4;
constexpr int kNormRowsPerBlock = 2 * (256 / kNormLanes);  // per block and step
template <int D, bool kX16>
__device__ __forceinline__ void row_norms(int64_t blk, int64_t nblk, const uint4* __restrict__ qk,
                                          float2* __restrict__ xnorm, float* __restrict__ knorm,
                                          int64_t N) {
  constexpr int kPieces = D / 8 / kNormLanes;      // 16-byte pieces per lane and row
  constexpr int kRowsPerBlock = 256 / kNormLanes;
  const int sub = threadIdx.x % kNormLanes;
  const int64_t stride = nblk * kRowsPerBlock;
  for (int64_t row0 = blk * kRowsPerBlock + threadIdx.x / kNormLanes; row0 < N;
       row0 += 2 * stride) {
    uint4 raw[2][kPieces];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t row = row0 + u * stride;
      const int64_t rc = row < N ? row : row0;
#pragma unroll
      for (int k = 0; k < kPieces; ++k) raw[u][k] = qk[rc * (D / 8) + k * kNormLanes + sub];
    }
    // The sums follow the projection epilogue's order (one piece per lane,
    // pairs combined by xor shuffles over 1, 2, 4, ...): per piece from 0,
    // then across the 4 lanes (pieces k*4 + 0..3), then the lane's pieces
    // pairwise, so both give the same bits.
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int64_t row = row0 + u * stride;
      float bk[kPieces], ck[kPieces];
#pragma unroll
      for (int k = 0; k < kPieces; ++k) {
        bk[k] = 0.f;
        ck[k] = 0.f;
        if (kX16) {
          hx::x16_piece(raw[u][k], bk[k], ck[k]);
        } else {
          const uint32_t wv[4] = {raw[u][k].x, raw[u][k].y, raw[u][k].z, raw[u][k].w};
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const float x0 = __uint_as_float(wv[q] << 16);
            const float x1 = __uint_as_float(wv[q] & 0xFFFF0000u);
            ck[k] = fmaf(x0, x0, fmaf(x1, x1, ck[k]));
          }
        }
#pragma unroll
        for (int off = 1; off < kNormLanes; off <<= 1) {
          ck[k] += __shfl_xor(ck[k], off);
          if (kX16) bk[k] += __shfl_xor(bk[k], off);
        }
      }
#pragma unroll
      for (int span = 1; span < kPieces; span <<= 1)
#pragma unroll
        for (int k = 0; k < kPieces; k += 2 * span) {
          ck[k] += ck[k + span];
          bk[k] += bk[k + span];
        }
      if (sub == 0 && row < N) {
        if (knorm) knorm[row] = ck[0];
        if (kX16) xnorm[row] = hx::norm_bounds(ck[0], bk[0]);
      }
    }
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_key_norms(const uint4* __restrict__ qk,
                                                   float* __restrict__ knorm, int64_t N) {
  row_norms<D, false>(blockIdx.x, gridDim.x, qk, nullptr, knorm, N);
}

// The hash's preparation in one launch: blocks 0 .. n_prep-1 prepare the
// rotation tiles, the others the row norms (none when the projection wrote
// them); the first of those clears the queue counters of this forward.
template <int D>
__global__ __launch_bounds__(256) void k_hash_prepare(
    const float* __restrict__ rot, _Float16* __restrict__ rh, float* __restrict__ rt,
    float4* __restrict__ part, const uint4* __restrict__ qk, float2* __restrict__ xnorm,
    float* __restrict__ knorm, int64_t N, unsigned* __restrict__ qcount, int d, int half,
    int half_pad, int n_prep) {
  if ((int)blockIdx.x < n_prep) {
    prep_tile(blockIdx.x, rot, rh, rt, part, d, half, half_pad);
    return;
  }
  if ((int)blockIdx.x == n_prep && threadIdx.x < 2) qcount[threadIdx.x] = 0u;
  row_norms<D, true>((int64_t)blockIdx.x - n_prep, (int64_t)gridDim.x - n_prep, qk, xnorm, knorm,
                     N);
}

struct QA {  // two-candidate re-score
  uint32_t row_lo, row_hi, k1, k2;
};
// Re-score entries are first appended to a workgroup queue in LDS (LDS atomics
// answer in tens of cycles) and moved to the global queues, one global atomic
// per queue, when the workgroup ends; only a full LDS queue appends globally.
// Each wave also keeps in LDS the tokens whose winner its main pass left
// open (kWq slots; rescanned 64 at a time).
constexpr int kQaLds = 256, kQbLds = 64, kWq = 128;
constexpr int kQueueLdsBytes = kQaLds * 16 + kQbLds * 8 + 16 + (kThreads / 64) * kWq * 4;

// Keep the two largest of (t1 >= t2) and keys a, b: max3 for the first; the
// second is the larger of t2 and the middle of (t1, a, b). (Keys order as
// floats like their bit patterns, see top3.)
__device__ __forceinline__ void top2_pair(uint32_t& t1, uint32_t& t2, uint32_t a, uint32_t b) {
  const uint32_t m = __float_as_uint(
      __builtin_amdgcn_fmed3f(__uint_as_float(t1), __uint_as_float(a), __uint_as_float(b)));
  const uint32_t n1 = t1 > a ? t1 : a;
  t1 = n1 > b ? n1 : b;
  t2 = t2 > m ? t2 : m;
}

template <bool B>
using Mode = std::integral_constant<bool, B>;

// Persistent: workgroup w serves round r and token tiles j = grp, grp + G/R, ...
// (tiles of kTokWG tokens). Its rotation R_r stays in LDS for the whole walk.
// w -> (xcd = w % 8, k = w / 8, r = k % R, grp = xcd + 8 (k / R)): the R
// workgroups that read the same token tile differ only in r and run on the
// same XCD, so the tile is fetched from HBM once and the other rounds find it
// in that XCD's L2.
//
// Every wave works on its own 64 tokens of a tile, in two modes. The main
// mode keeps the two largest keys per row (2.5 vector instructions per key):
// a row whose winner is certain gets its bucket, any other row's token goes
// to the wave's rescan queue in LDS. Whenever that queue holds 64 tokens, and
// once at the end of the walk, the wave runs the rescan mode on them: the
// same projections (bit for bit) keeping three keys per row, which decide
// between the certain winner, queue A (two candidates) and queue B (all
// columns).
template <int D>
__global__ __launch_bounds__(kThreads) void k_hash_mfma(
    const uint16_t* __restrict__ qkb, const float2* __restrict__ xnorm,
    const _Float16* __restrict__ rh,
    const float4* __restrict__ part, uint16_t* __restrict__ buckets,
    int32_t* __restrict__ buckets_out, QA* __restrict__ qa, uint2* __restrict__ qb,
    unsigned* __restrict__ qcount, int64_t N, int L, int R, int half, int half_pad, int ib,
    int n_tok_tiles) {
  constexpr int KS = D / 16;           // K-steps of 16
  constexpr int ROWB = 2 * D + 16;     // LDS bytes per rotation column
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hf = lane >> 5;            // which half of the dims this lane feeds
  const int tl = lane & 31;            // token within a set
  const uint32_t imask = (1u << ib) - 1u;
  const uint32_t vmask = 0x7FFFFFFFu & ~imask;
  // the key mask in a vector register: the key's index part is uniform and
  // takes the one scalar operand v_and_or_b32 may have
  uint32_t vmask_v;
  asm("v_mov_b32 %0, %1" : "=v"(vmask_v) : "s"(vmask));
  const float gamma = (float)(D + 2) * 1.1920928955078125e-07f;

  QA* qa_l = (QA*)(lds + half_pad * ROWB);
  uint2* qb_l = (uint2*)(lds + half_pad * ROWB + kQaLds * 16);
  unsigned* qn_l = (unsigned*)(lds + half_pad * ROWB + kQaLds * 16 + kQbLds * 8);
  uint32_t* wq = (uint32_t*)(lds + half_pad * ROWB + kQaLds * 16 + kQbLds * 8 + 16) + w * kWq;
  if (threadIdx.x < 2) qn_l[threadIdx.x] = 0u;
  int r, grp;
  walks::hash_block(blockIdx.x, R, r, grp);
  const int ngrp = gridDim.x / R;      // gridDim.x is a multiple of 8 R

  // x in fp16 as the B operand: lane half hf holds dims [hf*D/2, hf*D/2 + D/2)
  // of token tl of each set, K-step ks covering dims hf*D/2 + 8ks + 0..7 (the
  // K order of both operands is permuted the same way, which leaves the
  // product as is). A wave loads its token rows (bf16) when it starts a tile
  // (the other wave of its SIMD computes meanwhile) and converts them to
  // fp16 in registers (hx::x16_pair, 1.5 instructions per value); the first
  // tile's rows are loaded while the rotation is copied into LDS.
  uint4 bn[2][KS];
  float2 nn[2];
  auto load_rows = [&](uint4 (&b)[2][KS], float2 (&nrm)[2], const int64_t (&tok)[2]) {
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint4* src = (const uint4*)(qkb + tok[s] * D) + hf * KS;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) b[s][ks] = src[ks];
      nrm[s] = xnorm[tok[s]];
    }
  };
  auto to_f16 = [&](f16x8_t (&bx)[2][KS], const uint4 (&b)[2][KS]) {
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint32_t w[4] = {b[s][ks].x, b[s][ks].y, b[s][ks].z, b[s][ks].w};
        uint32_t h[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          float x0, x1;
          h[q] = hx::x16_pair(w[q], x0, x1);
        }
        bx[s][ks] = __builtin_bit_cast(f16x8_t, make_uint4(h[0], h[1], h[2], h[3]));
      }
  };
  auto fetch = [&](int j) {
    int64_t tok[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int64_t n = (int64_t)j * kTokWG + w * kTokWave + s * 32 + tl;
      tok[s] = n < N ? n : 0;
    }
    load_rows(bn, nn, tok);
  };
  if (grp < n_tok_tiles) fetch(grp);

  // rotation of round r -> LDS: every load of a thread in flight at once
  // (kRotLoads of 16 bytes cover 128 KB over the workgroup), then the stores
  {
    const uint4* g = (const uint4*)(rh + (int64_t)r * half_pad * D);
    const int total = half_pad * (D / 8);
    for (int base = threadIdx.x; base < total; base += kThreads * kRotLoads) {
      uint4 tmp[kRotLoads];
#pragma unroll
      for (int u = 0; u < kRotLoads; ++u) {
        const int idx = base + u * kThreads;
        tmp[u] = g[idx < total ? idx : 0];
      }
#pragma unroll
      for (int u = 0; u < kRotLoads; ++u) {
        const int idx = base + u * kThreads;
        if (idx < total) *(uint4*)(lds + (idx / (D / 8)) * ROWB + (idx % (D / 8)) * 16) = tmp[u];
      }
    }
  }
  __syncthreads();
  const int ntiles = half_pad / 32;
  float rh_max = 0.f, lo_max = 0.f, r_max = 0.f;  // over the round's column tiles
  for (int t = 0; t < ntiles; ++t) {
    const float4 b = part[r * ntiles + t];
    rh_max = fmaxf(rh_max, b.x);
    lo_max = fmaxf(lo_max, b.y);
    r_max = fmaxf(r_max, b.z);
  }

  // One wave's 64 tokens (2 sets of 32) against every column of the round.
  // Returns whether this lane's row (token tl of set hf) is left open (main
  // mode only). bh, i: the row's head and position.
  auto run = [&](auto mode, const f16x8_t (&bx)[2][KS], const float (&nx)[2],
                 const float (&nres)[2], bool valid, int64_t bh, int64_t i) -> bool {
    constexpr bool kT3 = decltype(mode)::value;
    // two independent key lists per set (even and odd accumulator
    // registers), merged once per token tile: half the dependency chain
    uint32_t t1[2] = {0u, 0u}, t2[2] = {0u, 0u}, t3[2] = {0u, 0u};
    uint32_t u1[2] = {0u, 0u}, u2[2] = {0u, 0u}, u3[2] = {0u, 0u};
    // Rotation tiles (the A operand, shared by both sets) are read from LDS
    // at the start of the step that multiplies them. A read past the last
    // tile re-reads the last one (never used).
    auto load_tile = [&](int kt, f16x8_t (&at)[KS]) {
      const int kc = kt < ntiles ? kt : ntiles - 1;
      const unsigned char* arow = lds + (kc * 32 + tl) * ROWB + hf * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) at[ks] = *(const f16x8_t*)(arow + ks * 16);
    };
    auto set_mfma = [&](floatx16_t& acc, int s, const f16x8_t (&at)[KS]) {
      const floatx16_t zero = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(at[ks], bx[s][ks], ks == 0 ? zero : acc, 0, 0, 0);
    };
    // C layout: lane holds token tl and columns kt*32 + 8(v/4) + 4 hf + v%4.
    // The index field gets kt*32 + 8(v/4) + v%4 (uniform across the wave); bit
    // 2 (the lane half) is added when the halves merge. Within one lane the
    // order of keys is the same with or without that bit.
    auto key = [&](int kt, const floatx16_t& c, int v) {
      // the tile's base index is opaque to the compiler, so the key's index
      // stays one scalar add and the key one v_and_or_b32 (not and + or3)
      uint32_t kb = (uint32_t)(kt * 32);
      asm("" : "+s"(kb));
      const uint32_t k = kb + (uint32_t)(8 * (v >> 2) + (v & 3));
      return (__float_as_uint(c[v]) & vmask_v) | k;
    };
    auto fold = [&](int kt, const floatx16_t& c, int s) {
      if constexpr (kT3) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          if (v & 1) top3(u1[s], u2[s], u3[s], key(kt, c, v));
          else top3(t1[s], t2[s], t3[s], key(kt, c, v));
        }
      } else {
        // pairs (v, v + 2): v = 0, 4, 8, 12 to the even list, 1, 5, 9, 13
        // to the odd one
#pragma unroll
        for (int v = 0; v < 16; v += 4) {
          top2_pair(t1[s], t2[s], key(kt, c, v), key(kt, c, v + 2));
          top2_pair(u1[s], u2[s], key(kt, c, v + 1), key(kt, c, v + 3));
        }
      }
    };
    // vector instructions per set, tile and MFMA: 4 per key for three keys,
    // about 2.5 for two
    constexpr int kFoldPerMfma = kT3 ? 8 : 5;
    // Tiles alternate between two accumulator pairs: each set's keys of tile
    // kt are folded from one pair while the MFMAs of tile kt + 1 fill the
    // other, so the fold reads the MFMA results in place (no copies). The
    // group barriers interleave one MFMA with the vector work around it.
    // one rotation tile buffer: tile kt + 1 is read at the start of step kt,
    // the fold of tile kt covering the read's latency
    f16x8_t at[KS];
    auto step = [&](int kt, floatx16_t (&cur)[2], floatx16_t (&nxt)[2]) {
      load_tile(kt + 1, at);
      set_mfma(nxt[0], 0, at);
      fold(kt, cur[0], 0);
      __builtin_amdgcn_sched_group_barrier(0x100, KS, 0);  // rotation tile reads
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kFoldPerMfma, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      set_mfma(nxt[1], 1, at);
      fold(kt, cur[1], 1);
      __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);
#pragma unroll
      for (int i = 0; i < KS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, kFoldPerMfma, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    floatx16_t even[2], odd[2];
    load_tile(0, at);
    set_mfma(even[0], 0, at);
    set_mfma(even[1], 1, at);
    int kt = 0;
    for (; kt + 2 < ntiles; kt += 2) {
      step(kt, even, odd);
      step(kt + 1, odd, even);
    }
    if (kt + 1 < ntiles) {
      step(kt, even, odd);
      fold(kt + 1, odd[0], 0);
      fold(kt + 1, odd[1], 1);
    } else {
      fold(kt, even[0], 0);
      fold(kt, even[1], 1);
    }
    // merge the odd list into the even one, then the two lane halves (same
    // tokens, other columns)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      if constexpr (kT3) {
        top3(t1[s], t2[s], t3[s], u1[s]);
        top3(t1[s], t2[s], t3[s], u2[s]);
        top3(t1[s], t2[s], t3[s], u3[s]);
        t1[s] |= (uint32_t)(hf << 2);
        t2[s] |= (uint32_t)(hf << 2);
        t3[s] |= (uint32_t)(hf << 2);
        const uint32_t o1 = __shfl_xor(t1[s], 32), o2 = __shfl_xor(t2[s], 32),
                       o3 = __shfl_xor(t3[s], 32);
        top3(t1[s], t2[s], t3[s], o1);
        top3(t1[s], t2[s], t3[s], o2);
        top3(t1[s], t2[s], t3[s], o3);
      } else {
        top2_pair(t1[s], t2[s], u1[s], u2[s]);
        t1[s] |= (uint32_t)(hf << 2);
        t2[s] |= (uint32_t)(hf << 2);
        const uint32_t o1 = __shfl_xor(t1[s], 32), o2 = __shfl_xor(t2[s], 32);
        top2_pair(t1[s], t2[s], o1, o2);
      }
    }
    // sign of p~ at each set's best column, partial over this lane's dims
    // (four partial sums: any fp32 order is within the certificate's bound)
    float part[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t k1 = t1[s] & imask;
      const unsigned char* row = lds + k1 * ROWB + hf * D;
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f16x8_t a = *(const f16x8_t*)(row + ks * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const f16x2_t pa = {a[2 * q], a[2 * q + 1]};
          const f16x2_t pb = {bx[s][ks][2 * q], bx[s][ks][2 * q + 1]};
          acc[q] = __builtin_amdgcn_fdot2(pa, pb, acc[q], false);
        }
      }
      part[s] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
    // this lane finishes set hf; the partner holds the other half of its dims
    const float send = hf ? part[0] : part[1];
    const float recv = __shfl_xor(send, 32);
    const float pk1 = (hf ? part[1] : part[0]) + recv;

    if (!valid) return false;
    const uint32_t a1 = hf ? t1[1] : t1[0];
    const uint32_t a2 = hf ? t2[1] : t2[0];
    const float d1 = __uint_as_float(a1 & vmask);
    const float d2 = __uint_as_float(a2 & vmask);
    const float ex = (gamma * rh_max + lo_max) * (hf ? nx[1] : nx[0]) +
                     r_max * (hf ? nres[1] : nres[0]);
    const float thr = 2.0f * (ex + ldexpf(d1, ib - 22));
    const int64_t row = (bh * R + r) * L + i;
    const uint32_t k1 = a1 & imask;
    if (d1 - d2 > thr && k1 < (uint32_t)half) {
      const int bk = (int)k1 + (pk1 < 0.f ? half : 0);
      buckets[row] = (uint16_t)bk;
      if (buckets_out) buckets_out[row] = bk;
      return false;
    }
    if constexpr (!kT3) {
      return true;
    } else {
      const uint32_t a3 = hf ? t3[1] : t3[0];
      const float d3 = __uint_as_float(a3 & vmask);
      if (d1 - d3 > thr && k1 < (uint32_t)half && (a2 & imask) < (uint32_t)half) {
        const QA entry{(uint32_t)row, (uint32_t)(row >> 32), k1, a2 & imask};
        const unsigned q = atomicAdd(qn_l + 0, 1u);
        if (q < (unsigned)kQaLds) qa_l[q] = entry;
        else qa[atomicAdd(qcount + 0, 1u)] = entry;
      } else {
        const uint2 entry = make_uint2((uint32_t)row, (uint32_t)(row >> 32));
        const unsigned q = atomicAdd(qn_l + 1, 1u);
        if (q < (unsigned)kQbLds) qb_l[q] = entry;
        else qb[atomicAdd(qcount + 1, 1u)] = entry;
      }
      return false;
    }
  };

  // rescan of the first c (<= 64) tokens of the wave's queue: token e of the
  // queue is token tl = e % 32 of set e / 32
  auto rescan = [&](unsigned c) {
    int64_t tok[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const unsigned e = (unsigned)(s * 32 + tl);
      tok[s] = e < c ? (int64_t)wq[e] : 0;
    }
    uint4 raw[2][KS];
    float2 nrm[2];
    load_rows(raw, nrm, tok);
    f16x8_t b[2][KS];
    to_f16(b, raw);
    const float nx[2] = {nrm[0].x, nrm[1].x}, nres[2] = {nrm[0].y, nrm[1].y};
    const int64_t n = hf ? tok[1] : tok[0];
    const int64_t bh = n / L;
    (void)run(Mode<true>(), b, nx, nres, (unsigned)(hf * 32 + tl) < c, bh, n - bh * L);
  };

  // head and position of the wave's first token (wave-uniform), advanced by
  // the walk's stride at the end of every token tile: one division per walk
  const int64_t tfirst = (int64_t)grp * kTokWG + __builtin_amdgcn_readfirstlane(w) * kTokWave;
  walks::TokenWalk tw;
  tw.init(tfirst, (int64_t)ngrp * kTokWG, L);
  const uint64_t below = (1ull << lane) - 1ull;
  unsigned nq = 0;  // tokens in the wave's rescan queue (wave-uniform)
  for (int j = grp; j < n_tok_tiles; j += ngrp) {
    const int64_t tok0 = (int64_t)j * kTokWG + w * kTokWave;
    if (j != grp) fetch(j);
    f16x8_t bx[2][KS];
    to_f16(bx, bn);
    float nx[2], nres[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      nx[s] = nn[s].x;
      nres[s] = nn[s].y;
    }
    const int64_t n = tok0 + hf * 32 + tl;
    int64_t bh, i;
    tw.at(hf * 32 + tl, bh, i);
    const bool open = run(Mode<false>(), bx, nx, nres, n < N, bh, i);
    // append the open rows' tokens to the wave's queue, in lane order
    const uint64_t m = __ballot(open);
    if (open) wq[nq + (unsigned)__popcll(m & below)] = (uint32_t)n;
    nq += (unsigned)__popcll(m);
    if (nq >= 64) {
      rescan(64);
      // the rest (fewer than 64) moves to the front
      const uint32_t rest = lane + 64 < (int)nq ? wq[64 + lane] : 0u;
      if (lane + 64 < (int)nq) wq[lane] = rest;
      nq -= 64;
    }
    tw.advance();
  }
  if (nq > 0) rescan(nq);
  // move the workgroup's queued entries to the global queues
  __syncthreads();
  unsigned* base_l = qn_l + 2;
  const unsigned na = min(qn_l[0], (unsigned)kQaLds), nb = min(qn_l[1], (unsigned)kQbLds);
  if (threadIdx.x == 0) {
    base_l[0] = na ? atomicAdd(qcount + 0, na) : 0u;
    base_l[1] = nb ? atomicAdd(qcount + 1, nb) : 0u;
  }
  __syncthreads();
  for (unsigned e = threadIdx.x; e < na; e += kThreads) qa[base_l[0] + e] = qa_l[e];
  for (unsigned e = threadIdx.x; e < nb; e += kThreads) qb[base_l[1] + e] = qb_l[e];
}

// Better of two (value, index) candidates under "largest value, lowest index".
__device__ __forceinline__ void take_better(double& v, int& k, double ov, int ok) {
  if (ov > v || (ov == v && ok < k)) {
    v = ov;
    k = ok;
  }
}

// Exact re-scoring of the rows the certificate could not settle, as the
// plain fp64 dot product with the sum over t = 0..d-1 in order (each product
// of a bf16 and an fp32 is exact in fp64), so the chosen bucket is the one the
// fp64 definition gives, tie rule included.
//  * queue B (all columns; rare): one workgroup per row, threads over
//    columns, reading the rotation in its own [r][t][k] layout (coalesced
//    over k) in batches of kQbT rows of t, x_t broadcast from the lane that
//    loaded it; the workgroup's best (value, column) is reduced through LDS.
//    Workgroups take these rows first.
//  * queue A (two candidates): one thread per (entry, candidate), the x row
//    and the candidate's column read straight from memory; the two threads of
//    an entry are neighbouring lanes and compare through a lane swap.
// Thread 0 of workgroup 0 also reports the queue sizes.
constexpr int kQbT = 32;  // rows of t whose loads are in flight together (x2 columns)
template <int D>
__global__ __launch_bounds__(256) void k_hash_fallback(const uint16_t* __restrict__ qk,
                                                       const float* __restrict__ rot,
                                                       const float* __restrict__ rt,
                                                       const QA* __restrict__ qa,
                                                       const uint2* __restrict__ qb,
                                                       const unsigned* __restrict__ qcount,
                                                       uint16_t* __restrict__ buckets,
                                                       int32_t* __restrict__ buckets_out,
                                                       unsigned long long* __restrict__ stats,
                                                       int L, int half, int R) {
  __shared__ double red_v[4];
  __shared__ int red_k[4];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  if (blockIdx.x == 0 && tid == 0) {
    stats[0] = qcount[0];
    stats[1] = qcount[1];
  }
  // queue B
  const int64_t nq = qcount[1];
  for (int64_t e = blockIdx.x; e < nq; e += gridDim.x) {
    const uint2 q = qb[e];
    const int64_t row = (int64_t)q.x | ((int64_t)q.y << 32);
    const int64_t seg = row / L, i = row - seg * L, bh = seg / R;
    const int r = (int)(seg - bh * R);
    const uint16_t* x = qk + (bh * L + i) * D;
    float xv[D / 64];
#pragma unroll
    for (int u = 0; u < D / 64; ++u) xv[u] = __uint_as_float((uint32_t)x[u * 64 + lane] << 16);
    const float* rr = rot + (int64_t)r * D * half;
    double best = -DBL_MAX;
    int bidx = INT_MAX;
    for (int k0 = 0; k0 < half; k0 += 512) {
      const int ka = k0 + tid, kb = k0 + 256 + tid;
      const int kca = ka < half ? ka : 0, kcb = kb < half ? kb : 0;
      double pa = 0.0, pb = 0.0;
      for (int t0 = 0; t0 < D; t0 += kQbT) {
        float ca[kQbT], cb[kQbT];
#pragma unroll
        for (int tt = 0; tt < kQbT; ++tt) {
          const float* rrow = rr + (int64_t)(t0 + tt) * half;
          ca[tt] = rrow[kca];
          cb[tt] = rrow[kcb];
        }
#pragma unroll
        for (int tt = 0; tt < kQbT; ++tt) {
          const int t = t0 + tt;
          const double xt = (double)__uint_as_float(
              __builtin_amdgcn_readlane(__float_as_uint(xv[t / 64]), t & 63));
          pa += xt * (double)ca[tt];
          pb += xt * (double)cb[tt];
        }
        __builtin_amdgcn_sched_group_barrier(0x020, 2 * kQbT, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, 1000, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      if (ka < half) {
        take_better(best, bidx, pa, ka);
        take_better(best, bidx, -pa, ka + half);
      }
      if (kb < half) {
        take_better(best, bidx, pb, kb);
        take_better(best, bidx, -pb, kb + half);
      }
    }
    for (int off = 32; off > 0; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int ok = __shfl_xor(bidx, off);
      take_better(best, bidx, ob, ok);
    }
    if (lane == 0) {
      red_v[wv] = best;
      red_k[wv] = bidx;
    }
    __syncthreads();
    if (tid == 0) {
      for (int u = 1; u < 4; ++u) take_better(best, bidx, red_v[u], red_k[u]);
      if (bidx < 0 || bidx >= 2 * half) bidx = 0;  // NaN input: keep the id in range
      buckets[row] = (uint16_t)bidx;
      if (buckets_out) buckets_out[row] = bidx;
    }
    __syncthreads();
  }
  // queue A
  const int64_t na2 = 2 * (int64_t)qcount[0];
  const int64_t stride = (int64_t)gridDim.x * 256;
  for (int64_t g = (int64_t)blockIdx.x * 256 + tid; g < na2; g += stride) {
    const QA q = qa[g >> 1];
    const int64_t row = (int64_t)q.row_lo | ((int64_t)q.row_hi << 32);
    const int k = (int)((g & 1) ? q.k2 : q.k1);
    const int64_t seg = row / L, i = row - seg * L, bh = seg / R;
    const int r = (int)(seg - bh * R);
    const uint4* xp = (const uint4*)(qk + (bh * L + i) * D);
    const float4* cp = (const float4*)(rt + ((int64_t)r * half + k) * D);
    uint4 xr[D / 8];
    float4 cr[D / 4];
#pragma unroll
    for (int u = 0; u < D / 8; ++u) xr[u] = xp[u];
#pragma unroll
    for (int u = 0; u < D / 4; ++u) cr[u] = cp[u];
    double p = 0.0;
#pragma unroll
    for (int u = 0; u < D / 8; ++u) {
      const uint32_t wq[4] = {xr[u].x, xr[u].y, xr[u].z, xr[u].w};
      const float cv[8] = {cr[2 * u].x, cr[2 * u].y, cr[2 * u].z, cr[2 * u].w,
                           cr[2 * u + 1].x, cr[2 * u + 1].y, cr[2 * u + 1].z, cr[2 * u + 1].w};
#pragma unroll
      for (int qd = 0; qd < 4; ++qd) {
        p += (double)__uint_as_float(wq[qd] << 16) * (double)cv[2 * qd];
        p += (double)__uint_as_float(wq[qd] & 0xFFFF0000u) * (double)cv[2 * qd + 1];
      }
    }
    double best = -DBL_MAX;
    int bidx = INT_MAX;
    take_better(best, bidx, p, k);
    take_better(best, bidx, -p, k + half);
    const double ob = __shfl_xor(best, 1);
    const int ok = __shfl_xor(bidx, 1);
    take_better(best, bidx, ob, ok);
    if ((g & 1) == 0) {
      buckets[row] = (uint16_t)bidx;
      if (buckets_out) buckets_out[row] = bidx;
    }
  }
}

template <int D>
constexpr int lds_bytes(int half_pad) { return half_pad * (2 * D + 16) + kQueueLdsBytes; }

int ceil_log2(int x) {
  int b = 0;
  while ((1 << b) < x) ++b;
  return b;
}

}  // namespace

int hash_half_pad(const Problem& p) { return ((p.half() + 31) / 32) * 32; }

hipError_t launch_key_norms(const Problem& p, const void* qk, float* knorm, hipStream_t s) {
  const int64_t N = p.n_token_heads();
  const int64_t want = (N + kNormRowsPerBlock - 1) / kNormRowsPerBlock;
  const unsigned blocks = (unsigned)(want < 65536 ? want : 65536);
  if (p.d == 128)
    hipLaunchKernelGGL(k_key_norms<128>, dim3(blocks), dim3(256), 0, s, (const uint4*)qk, knorm,
                       N);
  else
    hipLaunchKernelGGL(k_key_norms<64>, dim3(blocks), dim3(256), 0, s, (const uint4*)qk, knorm, N);
  return hipGetLastError();
}

bool hash_mfma_supported(const Problem& p) {
  if (p.dtype != LSH_ATTN_BF16 || p.nb < 2 || (p.d != 64 && p.d != 128)) return false;
  if (p.n_token_heads() >= ((int64_t)1 << 32)) return false;  // rescan queues hold u32 tokens
  const int hp = hash_half_pad(p);
  const int bytes = p.d == 64 ? lds_bytes<64>(hp) : lds_bytes<128>(hp);
  return bytes <= 150 * 1024;
}

hipError_t launch_hash_mfma(const Problem& p, const void* qk, const float* rot, HashScratch& hs,
                            uint16_t* buckets, int32_t* buckets_out, unsigned long long* stats,
                            float* knorm, hipStream_t s, hipEvent_t after_prep,
                            hipEvent_t after_main, bool norms_ready) {
  const int half = p.half();
  const int hp = hash_half_pad(p);
  const int ib = ceil_log2(hp) > 5 ? ceil_log2(hp) : 5;
  // hs.bounds: per (round, column tile) the rotation's partial maxima
  // (float4), then the counts of queues A and B
  const int n_prep = p.R * (hp / 32);
  float4* part = (float4*)hs.bounds;
  unsigned* qcount = hs.bounds + 4 * n_prep;
  const int64_t N = p.n_token_heads();
  const int n_tok_tiles = (int)((N + kTokWG - 1) / kTokWG);
  // persistent grid: as many resident workgroups as fit, a multiple of 8 R
  const int lds = p.d == 128 ? lds_bytes<128>(hp) : lds_bytes<64>(hp);
  const void* fn = p.d == 128 ? (const void*)k_hash_mfma<128> : (const void*)k_hash_mfma<64>;
  if (hs.per_cu == 0) {  // once per handle (on its device)
    (void)hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&hs.per_cu, fn, kThreads, lds) !=
            hipSuccess ||
        hs.per_cu < 1) {
      (void)hipGetLastError();
      hs.per_cu = 1;
    }
  }
  const int per_cu = hs.per_cu;
  const int64_t grid = walks::hash_grid(hs.n_cu, per_cu, p.R, n_tok_tiles);
  // rotation tiles and row norms (none when the projection wrote them) in one launch
  const int64_t n_rows = norms_ready ? 0 : N;
  const int64_t want = (n_rows + kNormRowsPerBlock - 1) / kNormRowsPerBlock;
  const unsigned blocks = (unsigned)(n_prep + (want < 1 ? 1 : want < 65536 ? want : 65536));
  if (p.d == 128)
    hipLaunchKernelGGL(k_hash_prepare<128>, dim3(blocks), dim3(256), 0, s, rot, hs.rh, hs.rt, part,
                       (const uint4*)qk, (float2*)hs.xnorm, knorm, n_rows, qcount, p.d, half, hp,
                       n_prep);
  else
    hipLaunchKernelGGL(k_hash_prepare<64>, dim3(blocks), dim3(256), 0, s, rot, hs.rh, hs.rt, part,
                       (const uint4*)qk, (float2*)hs.xnorm, knorm, n_rows, qcount, p.d, half, hp,
                       n_prep);
  if (after_prep) (void)hipEventRecord(after_prep, s);
  if (p.d == 128)
    hipLaunchKernelGGL(k_hash_mfma<128>, dim3((unsigned)grid), dim3(kThreads), lds, s,
                       (const uint16_t*)qk, (const float2*)hs.xnorm, hs.rh, part,
                       buckets, buckets_out,
                       (QA*)hs.queue_a, (uint2*)hs.queue_b, qcount, N, p.L, p.R, half, hp, ib,
                       n_tok_tiles);
  else
    hipLaunchKernelGGL(k_hash_mfma<64>, dim3((unsigned)grid), dim3(kThreads), lds, s,
                       (const uint16_t*)qk, (const float2*)hs.xnorm, hs.rh, part,
                       buckets, buckets_out,
                       (QA*)hs.queue_a, (uint2*)hs.queue_b, qcount, N, p.L, p.R, half, hp, ib,
                       n_tok_tiles);
  if (after_main) (void)hipEventRecord(after_main, s);
  if (p.d == 128)
    hipLaunchKernelGGL(k_hash_fallback<128>, dim3(1024), dim3(256), 0, s, (const uint16_t*)qk,
                       rot, hs.rt, (const QA*)hs.queue_a, (const uint2*)hs.queue_b, qcount, buckets,
                       buckets_out, stats, p.L, half, p.R);
  else
    hipLaunchKernelGGL(k_hash_fallback<64>, dim3(1024), dim3(256), 0, s, (const uint16_t*)qk,
                       rot, hs.rt, (const QA*)hs.queue_a, (const uint2*)hs.queue_b, qcount, buckets,
                       buckets_out, stats, p.L, half, p.R);
  return hipGetLastError();
}

}  // namespace lsh
