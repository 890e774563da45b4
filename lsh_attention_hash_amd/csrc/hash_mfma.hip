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
//  2. main: x (bf16) is rounded to fp16 the same way; v_mfma_f32_32x32x16_f16
//     gives p~ = x16 . Rh_k with exact products and fp32 sums. For every
//     column the kernel forms a key (bits of |p~| with the low ib mantissa bits
//     replaced by k) and keeps the three largest keys per row (max / med3).
//     With E = (gamma |Rh|max + |lo|max) |x16| + |R|max |x - x16| bounding
//     | |p~_k| - |p_k| | for every k (Cauchy-Schwarz on each correction term,
//     gamma = (d + 2) 2^-23 for the fp32 accumulation in any order) and S the
//     key truncation (2^(ib-22) of the top value):
//       top1 - top2 > 2 (E + S): the winner is certain; its sign comes from an
//         fp32 recomputation of p~_k1 (|p| > E, so the sign is right);
//       else top1 - top3 > 2 (E + S): only k1, k2 can win -> queue A;
//       else -> queue B (all columns).
//  3. fallback: queue A entries re-score the two candidates, queue B entries
//     every column, in fp64 with t = 0..d-1 in order: the products of a bf16
//     input and an fp32 rotation are exact in fp64, so these sums are the
//     correctly ordered fp64 projections, and the winner follows the rule of
//     the definition (largest entry, lowest index on ties).
#include <float.h>
#include <limits.h>

#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;     // 8 waves
constexpr int kTokWave = 64;      // 2 sets of 32 tokens per wave
constexpr int kTokWG = kThreads / 64 * kTokWave;
constexpr float kF16Max = 65504.0f;
constexpr float kF16MinNormal = 6.103515625e-05f;  // 2^-14

__device__ __forceinline__ float f16_round(float x) {
  const float c = fminf(fmaxf(x, -kF16Max), kF16Max);
  return fabsf(c) < kF16MinNormal ? 0.f : (float)(_Float16)c;
}

// upper bound of a non-negative double as float
__device__ __forceinline__ float up_f32(double x) { return (float)(x * (1.0 + 1e-6)) + 1e-30f; }

// One block of 64 threads per (round, padded column).
__global__ __launch_bounds__(64) void k_hash_prep(const float* __restrict__ rot,
                                                  _Float16* __restrict__ rh,
                                                  float* __restrict__ rt,
                                                  unsigned* __restrict__ bounds, int d, int half,
                                                  int half_pad) {
  const int k = blockIdx.x % (unsigned)half_pad;
  const int r = blockIdx.x / (unsigned)half_pad;
  const int t = threadIdx.x;
  double sh = 0.0, slo = 0.0, sr = 0.0;
  for (int u = t; u < d; u += 64) {
    const float x = k < half ? rot[((int64_t)r * d + u) * half + k] : 0.f;
    const float h = f16_round(x);
    rh[((int64_t)r * half_pad + k) * d + u] = (_Float16)h;
    if (k < half) rt[((int64_t)r * half + k) * d + u] = x;
    const double hd = h, xd = x;
    sh += hd * hd;
    slo += (xd - hd) * (xd - hd);
    sr += xd * xd;
  }
  for (int off = 32; off > 0; off >>= 1) {
    sh += __shfl_xor(sh, off);
    slo += __shfl_xor(slo, off);
    sr += __shfl_xor(sr, off);
  }
  if (t == 0) {
    // non-negative floats order like their bit patterns
    atomicMax(bounds + r * 4 + 0, __float_as_uint(up_f32(sqrt(sh))));
    atomicMax(bounds + r * 4 + 1, __float_as_uint(up_f32(sqrt(slo))));
    atomicMax(bounds + r * 4 + 2, __float_as_uint(up_f32(sqrt(sr))));
  }
}

__global__ void k_zero_u32(unsigned* p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0u;
}

// keep the three largest of (t1 >= t2 >= t3) and key
__device__ __forceinline__ void top3(uint32_t& t1, uint32_t& t2, uint32_t& t3, uint32_t key) {
  const uint32_t n1 = max(t1, key);
  const uint32_t n2 = max(t2, min(t1, key));  // median of (t1, t2, key), t1 >= t2
  const uint32_t n3 = max(t3, min(t2, key));
  t1 = n1;
  t2 = n2;
  t3 = n3;
}

struct QA {  // two-candidate re-score
  uint32_t row_lo, row_hi, k1, k2;
};

template <int D>
__global__ __launch_bounds__(kThreads) void k_hash_mfma(
    const uint16_t* __restrict__ qk, const _Float16* __restrict__ rh,
    const unsigned* __restrict__ bounds_u, uint16_t* __restrict__ buckets,
    int32_t* __restrict__ buckets_out, QA* __restrict__ qa, uint2* __restrict__ qb,
    unsigned* __restrict__ qcount, int64_t N, int L, int R, int half, int half_pad, int ib) {
  constexpr int KS = D / 16;           // K-steps of 16
  constexpr int ROWB = 2 * D + 16;     // LDS bytes per rotation column
  extern __shared__ __align__(16) unsigned char lds[];
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int hf = lane >> 5;            // which half of the dims this lane feeds
  const int tl = lane & 31;            // token within a set
  const int64_t tok0 = (int64_t)blockIdx.x * kTokWG + w * kTokWave;
  const uint32_t imask = (1u << ib) - 1u;
  const uint32_t vmask = 0x7FFFFFFFu & ~imask;
  const float gamma = (float)(D + 2) * 1.1920928955078125e-07f;

  // x in fp16 as the B operand: lane half hf holds dims [hf*D/2, hf*D/2 + D/2)
  // of token tl, K-step ks covering dims hf*D/2 + 8ks + 0..7 (the K order of
  // both operands is permuted the same way, which leaves the product as is)
  f16x8_t bx[2][KS];
  float nx[2], nres[2];
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const int64_t n = tok0 + s * 32 + tl;
    const bool valid = n < N;
    const uint4* src = (const uint4*)(qk + (valid ? n : 0) * D) + hf * KS;
    float a = 0.f, b = 0.f;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 raw = valid ? src[ks] : make_uint4(0, 0, 0, 0);
      const uint32_t wv[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float x0 = __uint_as_float(wv[j] << 16), x1 = __uint_as_float(wv[j] & 0xFFFF0000u);
        const float h0 = f16_round(x0), h1 = f16_round(x1);
        bx[s][ks][2 * j] = (_Float16)h0;
        bx[s][ks][2 * j + 1] = (_Float16)h1;
        a = fmaf(h0, h0, fmaf(h1, h1, a));
        b = fmaf(x0 - h0, x0 - h0, fmaf(x1 - h1, x1 - h1, b));
      }
    }
    a += __shfl_xor(a, 32);
    b += __shfl_xor(b, 32);
    nx[s] = sqrtf(a) * (1.0f + 1e-5f);
    nres[s] = sqrtf(b) * (1.0f + 1e-5f);
  }

  const int ntiles = half_pad / 32;
  for (int r = 0; r < R; ++r) {
    __syncthreads();
    {
      const uint4* g = (const uint4*)(rh + (int64_t)r * half_pad * D);
      for (int idx = threadIdx.x; idx < half_pad * (D / 8); idx += kThreads) {
        const int row = idx / (D / 8), c = idx % (D / 8);
        *(uint4*)(lds + row * ROWB + c * 16) = g[idx];
      }
    }
    __syncthreads();
    const float rh_max = __uint_as_float(bounds_u[r * 4 + 0]);
    const float lo_max = __uint_as_float(bounds_u[r * 4 + 1]);
    const float r_max = __uint_as_float(bounds_u[r * 4 + 2]);

    uint32_t t1[2] = {0u, 0u}, t2[2] = {0u, 0u}, t3[2] = {0u, 0u};
    for (int kt = 0; kt < ntiles; ++kt) {
      floatx16_t acc[2];
#pragma unroll
      for (int s = 0; s < 2; ++s)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[s][v] = 0.f;
      const unsigned char* arow = lds + (kt * 32 + tl) * ROWB + hf * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f16x8_t a = *(const f16x8_t*)(arow + ks * 16);
#pragma unroll
        for (int s = 0; s < 2; ++s)
          acc[s] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, bx[s][ks], acc[s], 0, 0, 0);
      }
      // C layout: lane holds token tl and columns kt*32 + 8(v/4) + 4 hf + v%4
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const uint32_t k = (uint32_t)(kt * 32 + 8 * (v >> 2) + 4 * hf + (v & 3));
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const uint32_t key = (__float_as_uint(acc[s][v]) & vmask) | k;
          top3(t1[s], t2[s], t3[s], key);
        }
      }
    }
    // merge the two lane halves (same tokens, other columns)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t o1 = __shfl_xor(t1[s], 32), o2 = __shfl_xor(t2[s], 32),
                     o3 = __shfl_xor(t3[s], 32);
      top3(t1[s], t2[s], t3[s], o1);
      top3(t1[s], t2[s], t3[s], o2);
      top3(t1[s], t2[s], t3[s], o3);
    }
    // sign of p~ at each set's best column, partial over this lane's dims
    float part[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const uint32_t k1 = t1[s] & imask;
      const unsigned char* row = lds + k1 * ROWB + hf * D;
      float acc = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const f16x8_t a = *(const f16x8_t*)(row + ks * 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f16x2_t pa = {a[2 * j], a[2 * j + 1]};
          const f16x2_t pb = {bx[s][ks][2 * j], bx[s][ks][2 * j + 1]};
          acc = __builtin_amdgcn_fdot2(pa, pb, acc, false);
        }
      }
      part[s] = acc;
    }
    // this lane finishes set hf; the partner holds the other half of its dims
    const float send = hf ? part[0] : part[1];
    const float recv = __shfl_xor(send, 32);
    const float pk1 = (hf ? part[1] : part[0]) + recv;

    const int s = hf;
    const int64_t n = tok0 + s * 32 + tl;
    if (n < N) {
      const uint32_t a1 = hf ? t1[1] : t1[0];
      const uint32_t a2 = hf ? t2[1] : t2[0];
      const uint32_t a3 = hf ? t3[1] : t3[0];
      const float d1 = __uint_as_float(a1 & vmask);
      const float d2 = __uint_as_float(a2 & vmask);
      const float d3 = __uint_as_float(a3 & vmask);
      const float ex = (gamma * rh_max + lo_max) * (hf ? nx[1] : nx[0]) +
                       r_max * (hf ? nres[1] : nres[0]);
      const float thr = 2.0f * (ex + ldexpf(d1, ib - 22));
      const int64_t bh = n / L;
      const int64_t i = n - bh * L;
      const int64_t row = (bh * R + r) * L + i;
      const uint32_t k1 = a1 & imask;
      if (d1 - d2 > thr && k1 < (uint32_t)half) {
        const int bk = (int)k1 + (pk1 < 0.f ? half : 0);
        buckets[row] = (uint16_t)bk;
        if (buckets_out) buckets_out[row] = bk;
      } else if (d1 - d3 > thr && k1 < (uint32_t)half && (a2 & imask) < (uint32_t)half) {
        const unsigned e = atomicAdd(qcount + 0, 1u);
        qa[e] = QA{(uint32_t)row, (uint32_t)(row >> 32), k1, a2 & imask};
      } else {
        const unsigned e = atomicAdd(qcount + 1, 1u);
        qb[e] = make_uint2((uint32_t)row, (uint32_t)(row >> 32));
      }
    }
  }
}

// Better of two (value, index) candidates under "largest value, lowest index".
__device__ __forceinline__ void take_better(double& v, int& k, double ov, int ok) {
  if (ov > v || (ov == v && ok < k)) {
    v = ov;
    k = ok;
  }
}

// fp64 projection of row x on column k, t = 0..d-1 in order
template <typename T>
__device__ __forceinline__ double proj64(const T* x, const float* rtk, int d) {
  double p = 0.0;
  for (int t = 0; t < d; ++t) p += (double)to_f32(x[t]) * (double)rtk[t];
  return p;
}

template <typename T>
__global__ __launch_bounds__(256) void k_hash_fallback(const T* __restrict__ qk,
                                                       const float* __restrict__ rt,
                                                       const QA* __restrict__ qa,
                                                       const uint2* __restrict__ qb,
                                                       const unsigned* __restrict__ qcount,
                                                       uint16_t* __restrict__ buckets,
                                                       int32_t* __restrict__ buckets_out, int L,
                                                       int d, int half, int R) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = (int64_t)blockIdx.x * (blockDim.x / 64) + threadIdx.x / 64;
  const int64_t waves = (int64_t)gridDim.x * (blockDim.x / 64);
  // queue A: 32 entries per wave, one lane per candidate
  const int64_t na = qcount[0];
  for (int64_t e0 = wave * 32; e0 < na; e0 += waves * 32) {
    const int64_t e = e0 + lane / 2;
    double best = -DBL_MAX;
    int bidx = INT_MAX;
    int64_t row = 0;
    if (e < na) {
      const QA q = qa[e];
      row = (int64_t)q.row_lo | ((int64_t)q.row_hi << 32);
      const int k = (lane & 1) ? (int)q.k2 : (int)q.k1;
      const int64_t seg = row / L, i = row - seg * L, bh = seg / R;
      const int r = (int)(seg - bh * R);
      const double p = proj64(qk + (bh * L + i) * d, rt + ((int64_t)r * half + k) * d, d);
      take_better(best, bidx, p, k);
      take_better(best, bidx, -p, k + half);
    }
    const double ob = __shfl_xor(best, 1);
    const int ok = __shfl_xor(bidx, 1);
    take_better(best, bidx, ob, ok);
    if (e < na && (lane & 1) == 0) {
      buckets[row] = (uint16_t)bidx;
      if (buckets_out) buckets_out[row] = bidx;
    }
  }
  // queue B: one wave per entry, lanes over columns
  const int64_t nb_ = qcount[1];
  for (int64_t e = wave; e < nb_; e += waves) {
    const uint2 q = qb[e];
    const int64_t row = (int64_t)q.x | ((int64_t)q.y << 32);
    const int64_t seg = row / L, i = row - seg * L, bh = seg / R;
    const int r = (int)(seg - bh * R);
    const T* x = qk + (bh * L + i) * d;
    double best = -DBL_MAX;
    int bidx = INT_MAX;
    for (int k = lane; k < half; k += 64) {
      const double p = proj64(x, rt + ((int64_t)r * half + k) * d, d);
      take_better(best, bidx, p, k);
      take_better(best, bidx, -p, k + half);
    }
    for (int off = 32; off > 0; off >>= 1) {
      const double ob = __shfl_xor(best, off);
      const int ok = __shfl_xor(bidx, off);
      take_better(best, bidx, ob, ok);
    }
    if (bidx < 0 || bidx >= 2 * half) bidx = 0;  // NaN input: keep the id in range
    if (lane == 0) {
      buckets[row] = (uint16_t)bidx;
      if (buckets_out) buckets_out[row] = bidx;
    }
  }
}

__global__ void k_hash_stats(const unsigned* __restrict__ qcount,
                             unsigned long long* __restrict__ stats) {
  if (threadIdx.x == 0) {
    stats[0] = qcount[0];
    stats[1] = qcount[1];
  }
}

template <int D>
constexpr int lds_bytes(int half_pad) { return half_pad * (2 * D + 16); }

int ceil_log2(int x) {
  int b = 0;
  while ((1 << b) < x) ++b;
  return b;
}

}  // namespace

int hash_half_pad(const Problem& p) { return ((p.half() + 31) / 32) * 32; }

bool hash_mfma_supported(const Problem& p) {
  if (p.dtype != LSH_ATTN_BF16 || p.nb < 2 || (p.d != 64 && p.d != 128)) return false;
  const int hp = hash_half_pad(p);
  const int bytes = p.d == 64 ? lds_bytes<64>(hp) : lds_bytes<128>(hp);
  return bytes <= 150 * 1024;
}

hipError_t launch_hash_mfma(const Problem& p, const void* qk, const float* rot, HashScratch& hs,
                            uint16_t* buckets, int32_t* buckets_out, unsigned long long* stats,
                            hipStream_t s) {
  const int half = p.half();
  const int hp = hash_half_pad(p);
  const int ib = ceil_log2(hp) > 5 ? ceil_log2(hp) : 5;
  hipLaunchKernelGGL(k_zero_u32, dim3(1), dim3(64), 0, s, hs.bounds, 4 * p.R + 2);
  unsigned* qcount = hs.bounds + 4 * p.R;
  hipLaunchKernelGGL(k_hash_prep, dim3((unsigned)(p.R * hp)), dim3(64), 0, s, rot, hs.rh, hs.rt,
                     hs.bounds, p.d, half, hp);
  const int64_t N = p.n_token_heads();
  const unsigned grid = (unsigned)((N + kTokWG - 1) / kTokWG);
  if (p.d == 128) {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)k_hash_mfma<128>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, 150 * 1024);
      attr = true;
    }
    hipLaunchKernelGGL(k_hash_mfma<128>, dim3(grid), dim3(kThreads), lds_bytes<128>(hp), s,
                       (const uint16_t*)qk, hs.rh, hs.bounds, buckets, buckets_out,
                       (QA*)hs.queue_a, (uint2*)hs.queue_b, qcount, N, p.L, p.R, half, hp, ib);
  } else {
    static bool attr = false;
    if (!attr) {
      (void)hipFuncSetAttribute((const void*)k_hash_mfma<64>, hipFuncAttributeMaxDynamicSharedMemorySize,
                          150 * 1024);
      attr = true;
    }
    hipLaunchKernelGGL(k_hash_mfma<64>, dim3(grid), dim3(kThreads), lds_bytes<64>(hp), s,
                       (const uint16_t*)qk, hs.rh, hs.bounds, buckets, buckets_out,
                       (QA*)hs.queue_a, (uint2*)hs.queue_b, qcount, N, p.L, p.R, half, hp, ib);
  }
  hipLaunchKernelGGL(k_hash_fallback<bf16_t>, dim3(1024), dim3(256), 0, s, (const bf16_t*)qk,
                     hs.rt, (const QA*)hs.queue_a, (const uint2*)hs.queue_b, qcount, buckets,
                     buckets_out, p.L, p.d, half, p.R);
  hipLaunchKernelGGL(k_hash_stats, dim3(1), dim3(64), 0, s, qcount, stats);
  return hipGetLastError();
}

}  // namespace lsh
