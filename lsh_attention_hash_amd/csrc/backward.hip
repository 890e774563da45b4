// backward.hip -- gradients of qk and v at the buckets of a forward.
//
// The hash (an argmax) and the sort (a permutation) are piecewise constant,
// so the gradient flows only through the chunk attention and the round
// combination, which are taken as in the forward (Reformer summary at
// p2.ttnews.xyz, LSH attention, multi-round and shared-QK sections; overview
// at www.dtcms.com/a/488796.html, section 2.1: unit keys, 1/sqrt(d) scale).
// With w_r(i) the combination weight of round r at position i, out(i) the
// combined output and P the round's softmax over a query's window, the chain
// rule through out = sum_r w_r o_r, w = softmax_r(lse_r) and the softmax gives,
// for an attendable key j of query i in round r:
//   dS_ij = w_r(i) P_ij (dout(i) . v_j - dout(i) . out(i))
// (the logsumexp's own term w_r (o_r - out) . dout and the softmax's
// dout . o_r term leave only dout . out), and with s_ij = q_i . khat_j / sqrt(d):
//   dq_i    = sum_j dS_ij khat_j / sqrt(d)
//   dkhat_j = sum_i dS_ij q_i / sqrt(d),   dv_j = sum_i w_r(i) P_ij dout(i).
// A query that saw only itself in round r has o_r(i) = v_i: it passes
// w_r(i) dout(i) to v_i. Key normalisation khat = k / |k| (0 for k = 0):
//   dk_j = (dkhat_j - khat_j (khat_j . dkhat_j)) / |k_j|,  dqk = dq + dk.
//
// On the matrix-core path (bf16, chunk_len 64, d in {64, 128}) the dq and
// (dkhat, dv) products run in one kernel of backward_mfma.hip instead of the
// two below; it also applies the normalisation per round, so its reduction
// (k_bwd_reduce_sum) only sums.
// Launches (one stream): the per-round attention is recomputed from the
// forward's permutation (fp32 rows and logsumexps; on the matrix-core path only
// the logsumexps and dout . o_r per query); per position, the round weights
// and dout . out; per round, dq of every query and dkhat, dv of every
// key (each key is seen by the queries of its chunk and of the next one); then
// the sum over rounds with the normalisation, in the caller's dtype. Every
// output element is written by one thread: no atomics, deterministic.
#include <type_traits>

#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* x);
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* x) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
template <>
__device__ __forceinline__ void load8<bf16_t>(const bf16_t* p, float* x) {
  const uint4 a = *(const uint4*)p;
  const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[2 * j] = __uint_as_float(w[j] << 16);
    x[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void store8(float* p, const float* x) {
  *(float4*)p = make_float4(x[0], x[1], x[2], x[3]);
  *(float4*)(p + 4) = make_float4(x[4], x[5], x[6], x[7]);
}
__device__ __forceinline__ void store8(bf16_t* p, const float* x) {
  uint32_t u[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    u[j] = (uint32_t)f32_to_bf16(x[2 * j]).bits | ((uint32_t)f32_to_bf16(x[2 * j + 1]).bits << 16);
  *(uint4*)p = make_uint4(u[0], u[1], u[2], u[3]);
}

// Sum over the kLpr lanes of one row (consecutive lanes, kLpr a power of two).
template <int kLpr>
__device__ __forceinline__ float row_sum(float x) {
#pragma unroll
  for (int off = 1; off < kLpr; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

__device__ __forceinline__ float dot8(const float* a, const float* b) {
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s = fmaf(a[u], b[u], s);
  return s;
}

// Per position (b, h, i): the round weights w_r(i) -> w [seg, L] and
// dout(i) . out(i) -> cq [bh, L], out recomputed from the fp32 round rows (v_i
// for a round in which the position saw only itself). D/8 lanes per row.
template <int D, typename T>
__global__ __launch_bounds__(256) void k_bwd_rows(const float* __restrict__ o,
                                                  const float* __restrict__ lse,
                                                  const T* __restrict__ v,
                                                  const T* __restrict__ dout,
                                                  float* __restrict__ w, float* __restrict__ cq,
                                                  int L, int R, int64_t o_seg_rows,
                                                  int64_t n_rows) {
  constexpr int kLpr = D / 8;
  const int sub = threadIdx.x % kLpr;
  const int64_t row = (int64_t)blockIdx.x * (256 / kLpr) + threadIdx.x / kLpr;
  if (row >= n_rows) return;
  const int64_t bh = row / L, i = row - bh * L;
  const float* lr = lse + bh * R * L + i;
  float mx = -INFINITY;
  for (int r = 0; r < R; ++r) mx = fmaxf(mx, lr[(int64_t)r * L]);
  float sum = 0.f;
  for (int r = 0; r < R; ++r) sum += __expf(lr[(int64_t)r * L] - mx);
  const float inv = 1.0f / sum;
  float vi[8], acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  load8<T>(v + row * D + sub * 8, vi);
  for (int r = 0; r < R; ++r) {
    const float l = lr[(int64_t)r * L];
    const float wr = __expf(l - mx) * inv;
    if (sub == 0) w[(bh * R + r) * L + i] = wr;
    float x[8];
    if (l == kSelfLogit) {
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = vi[u];
    } else {
      load8<float>(o + ((bh * R + r) * o_seg_rows + i) * D + sub * 8, x);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) acc[u] = fmaf(wr, x[u], acc[u]);
  }
  float dz[8];
  load8<T>(dout + row * D + sub * 8, dz);
  const float c = row_sum<kLpr>(dot8(dz, acc));
  if (sub == 0) cq[row] = c;
}

// As k_bwd_rows, from the per-round scalars od_r(i) = dout(i) . o_r(i) of the
// matrix-core recomputation (dout(i) . v_i for a round in which the position
// saw only itself): dout . out = sum_r w_r od_r. Also the summed weight of the
// self-only rounds per position, wself [B*H, L]. One thread per position.
__global__ __launch_bounds__(256) void k_bwd_rows_dot(const float* __restrict__ od,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ w,
                                                      float* __restrict__ cq,
                                                      float* __restrict__ wself, int L, int R,
                                                      int64_t n_rows) {
  const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (row >= n_rows) return;
  const int64_t bh = row / L, i = row - bh * L;
  const float* lr = lse + bh * R * L + i;
  const float* dr = od + bh * R * L + i;
  float mx = -INFINITY;
  for (int r = 0; r < R; ++r) mx = fmaxf(mx, lr[(int64_t)r * L]);
  float sum = 0.f;
  for (int r = 0; r < R; ++r) sum += __expf(lr[(int64_t)r * L] - mx);
  const float inv = 1.0f / sum;
  float c = 0.f, ws = 0.f;
  for (int r = 0; r < R; ++r) {
    const float l = lr[(int64_t)r * L];
    const float wr = __expf(l - mx) * inv;
    w[(bh * R + r) * L + i] = wr;
    c = fmaf(wr, dr[(int64_t)r * L], c);
    ws += l == kSelfLogit ? wr : 0.f;
  }
  cq[row] = c;
  wself[row] = ws;
}

// dq of the query at slot s of segment seg (one D/8-lane row group per
// query): the sum over its window of dS_ij khat_j / sqrt(d).
template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(256) void k_bwd_dq(const T* __restrict__ qk, const T* __restrict__ v,
                                                const T* __restrict__ dout,
                                                const int32_t* __restrict__ perm,
                                                const float* __restrict__ lse,
                                                const float* __restrict__ w,
                                                const float* __restrict__ cq,
                                                float* __restrict__ dq, int L, int m, int R,
                                                int64_t n_rows) {
  constexpr int kLpr = D / 8;
  const int sub = threadIdx.x % kLpr;
  const int64_t slot_row = (int64_t)blockIdx.x * (256 / kLpr) + threadIdx.x / kLpr;
  if (slot_row >= n_rows) return;
  const int64_t seg = slot_row / L;
  const int s = (int)(slot_row - seg * L);
  const int64_t bh = seg / R;
  const int32_t* pm = perm + seg * L;
  const int i = pm[s];
  const float l = lse[seg * L + i];
  float g[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (l != kSelfLogit) {
    const float scale = 1.0f / sqrtf((float)D);
    const float wi = w[seg * L + i], ci = cq[bh * L + i];
    float q[8], dz[8];
    load8<T>(qk + (bh * L + i) * D + sub * 8, q);
    load8<T>(dout + (bh * L + i) * D + sub * 8, dz);
    const int chunk = s / m;
    const int first = (chunk > 0 ? chunk - 1 : chunk) * m, last = (chunk + 1) * m;
    for (int t = first; t < last; ++t) {
      const int j = pm[t];
      if (j == i || (CAUSAL && j > i)) continue;
      float k[8], vj[8];
      load8<T>(qk + (bh * L + j) * D + sub * 8, k);
      load8<T>(v + (bh * L + j) * D + sub * 8, vj);
      const float n2 = row_sum<kLpr>(dot8(k, k));
      const float qkd = row_sum<kLpr>(dot8(q, k));
      const float dv = row_sum<kLpr>(dot8(dz, vj));
      const float rn = n2 > 0.f ? 1.0f / sqrtf(n2) : 0.f;
      const float p = __expf(qkd * rn * scale - l);
      const float ds = wi * p * (dv - ci);
#pragma unroll
      for (int u = 0; u < 8; ++u) g[u] = fmaf(ds * rn * scale, k[u], g[u]);
    }
  }
  store8(dq + (seg * L + i) * D + sub * 8, g);
}

// dkhat and dv of the key at slot t of segment seg: the queries that see it
// are those of its chunk and of the next one.
template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(256) void k_bwd_dkv(const T* __restrict__ qk, const T* __restrict__ v,
                                                 const T* __restrict__ dout,
                                                 const int32_t* __restrict__ perm,
                                                 const float* __restrict__ lse,
                                                 const float* __restrict__ w,
                                                 const float* __restrict__ cq,
                                                 float* __restrict__ dk, float* __restrict__ dv,
                                                 int L, int m, int R, int64_t n_rows) {
  constexpr int kLpr = D / 8;
  const int sub = threadIdx.x % kLpr;
  const int64_t slot_row = (int64_t)blockIdx.x * (256 / kLpr) + threadIdx.x / kLpr;
  if (slot_row >= n_rows) return;
  const int64_t seg = slot_row / L;
  const int t = (int)(slot_row - seg * L);
  const int64_t bh = seg / R;
  const int32_t* pm = perm + seg * L;
  const int j = pm[t];
  const float scale = 1.0f / sqrtf((float)D);
  float k[8], vj[8];
  load8<T>(qk + (bh * L + j) * D + sub * 8, k);
  load8<T>(v + (bh * L + j) * D + sub * 8, vj);
  const float n2 = row_sum<kLpr>(dot8(k, k));
  const float rn = n2 > 0.f ? 1.0f / sqrtf(n2) : 0.f;
  float gk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float gv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const int chunk = t / m;
  const int first = chunk * m, last = min(L, (chunk + 2) * m);
  for (int s = first; s < last; ++s) {
    const int i = pm[s];
    if (i == j || (CAUSAL && j > i)) continue;
    const float l = lse[seg * L + i];
    if (l == kSelfLogit) continue;
    const float wi = w[seg * L + i], ci = cq[bh * L + i];
    float q[8], dz[8];
    load8<T>(qk + (bh * L + i) * D + sub * 8, q);
    load8<T>(dout + (bh * L + i) * D + sub * 8, dz);
    const float qkd = row_sum<kLpr>(dot8(q, k));
    const float dvd = row_sum<kLpr>(dot8(dz, vj));
    const float p = __expf(qkd * rn * scale - l);
    const float ds = wi * p * (dvd - ci);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      gk[u] = fmaf(ds * scale, q[u], gk[u]);
      gv[u] = fmaf(wi * p, dz[u], gv[u]);
    }
  }
  store8(dk + (seg * L + j) * D + sub * 8, gk);
  store8(dv + (seg * L + j) * D + sub * 8, gv);
}

// Sum over rounds, key normalisation, the self-only value terms; dqk and dv
// in the caller's dtype. D/8 lanes per (b, h, position).
template <int D, typename T>
__global__ __launch_bounds__(256) void k_bwd_reduce(const T* __restrict__ qk,
                                                    const T* __restrict__ dout,
                                                    const float* __restrict__ lse,
                                                    const float* __restrict__ w,
                                                    const float* __restrict__ dq,
                                                    const float* __restrict__ dk,
                                                    const float* __restrict__ dvr,
                                                    T* __restrict__ dqk, T* __restrict__ dv,
                                                    int L, int R, int64_t n_rows) {
  constexpr int kLpr = D / 8;
  const int sub = threadIdx.x % kLpr;
  const int64_t row = (int64_t)blockIdx.x * (256 / kLpr) + threadIdx.x / kLpr;
  if (row >= n_rows) return;
  const int64_t bh = row / L, j = row - bh * L;
  float gq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float gk[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float gv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float wself = 0.f;
  for (int r = 0; r < R; ++r) {
    const int64_t sr = (bh * R + r) * L + j;
    float a[8], b[8], c[8];
    load8<float>(dq + sr * D + sub * 8, a);
    load8<float>(dk + sr * D + sub * 8, b);
    load8<float>(dvr + sr * D + sub * 8, c);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      gq[u] += a[u];
      gk[u] += b[u];
      gv[u] += c[u];
    }
    if (lse[sr] == kSelfLogit) wself += w[sr];
  }
  float k[8], dz[8];
  load8<T>(qk + row * D + sub * 8, k);
  load8<T>(dout + row * D + sub * 8, dz);
  const float n2 = row_sum<kLpr>(dot8(k, k));
  const float rn = n2 > 0.f ? 1.0f / sqrtf(n2) : 0.f;
  const float proj = row_sum<kLpr>(dot8(k, gk)) * rn;  // khat . dkhat
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    gq[u] += (gk[u] - k[u] * rn * proj) * rn;
    gv[u] = fmaf(wself, dz[u], gv[u]);
  }
  store8(dqk + row * D + sub * 8, gq);
  store8(dv + row * D + sub * 8, gv);
}

// The same on the matrix-core path, whose per-round rows (GT: fp16 or fp32)
// already hold dq + the normalised key gradient (dqk_r) and dv_r: sums over
// rounds in fp32 plus the self-only value term wself dout. kR > 0: R == kR
// and every load is issued before the sums; kR == 0: any R. Each per-round row
// is read once (non-temporal); blocks take the rows from the end, which the
// product kernel wrote last.
template <int D, typename T, int kR, typename GT>
__global__ __launch_bounds__(256) void k_bwd_reduce_sum(const T* __restrict__ dout,
                                                        const float* __restrict__ wself,
                                                        const GT* __restrict__ dqkr,
                                                        const GT* __restrict__ dvr,
                                                        T* __restrict__ dqk, T* __restrict__ dv,
                                                        int L, int R_rt, int64_t n_rows) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
  constexpr int kLpr = D / 8;
  constexpr int kG = kR > 0 ? kR : 1;
  const int R = kR > 0 ? kR : R_rt;
  const int sub = threadIdx.x % kLpr;
  const int64_t row = (int64_t)(gridDim.x - 1 - blockIdx.x) * (256 / kLpr) + threadIdx.x / kLpr;
  if (row >= n_rows) return;
  const int64_t bh = row / L, j = row - bh * L;
  float gq[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float gv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const float ws = wself[row];
  for (int r0 = 0; r0 < R; r0 += kG) {
    if constexpr (sizeof(GT) == 4) {
      f32x4_t a[kG][2], c[kG][2];
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int64_t sr = (bh * R + r0 + u) * L + j;
        const f32x4_t* pa = (const f32x4_t*)(dqkr + sr * D + sub * 8);
        const f32x4_t* pc = (const f32x4_t*)(dvr + sr * D + sub * 8);
        a[u][0] = __builtin_nontemporal_load(pa);
        a[u][1] = __builtin_nontemporal_load(pa + 1);
        c[u][0] = __builtin_nontemporal_load(pc);
        c[u][1] = __builtin_nontemporal_load(pc + 1);
      }
#pragma unroll
      for (int u = 0; u < kG; ++u)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          gq[k] += a[u][0][k];
          gq[4 + k] += a[u][1][k];
          gv[k] += c[u][0][k];
          gv[4 + k] += c[u][1][k];
        }
    } else {
      h8_t a[kG], c[kG];
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const int64_t sr = (bh * R + r0 + u) * L + j;
        a[u] = __builtin_nontemporal_load((const h8_t*)(dqkr + sr * D + sub * 8));
        c[u] = __builtin_nontemporal_load((const h8_t*)(dvr + sr * D + sub * 8));
      }
#pragma unroll
      for (int u = 0; u < kG; ++u)
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          gq[k] += (float)a[u][k];
          gv[k] += (float)c[u][k];
        }
    }
  }
  if (ws > 0.f) {
    float dz[8];
    load8<T>(dout + row * D + sub * 8, dz);
#pragma unroll
    for (int u = 0; u < 8; ++u) gv[u] = fmaf(ws, dz[u], gv[u]);
  }
  store8(dqk + row * D + sub * 8, gq);
  store8(dv + row * D + sub * 8, gv);
}

template <int D, typename T>
void launch_t(const Problem& p, const void* qk, const void* v, const int32_t* perm,
              const void* dout, void* dqk, void* dvo, const float* knorm, BwdWorkspace& b,
              hipStream_t s, const hipEvent_t* ev) {
  auto mark = [&](int j) {
    if (ev) (void)hipEventRecord(ev[j], s);
  };
  const int64_t rpb = 256 / (D / 8);
  const int64_t nt = p.n_token_heads(), nr = p.n_rows();
  const dim3 gt((unsigned)((nt + rpb - 1) / rpb)), gr((unsigned)((nr + rpb - 1) / rpb));
  if (attend_mfma_supported(p))
    hipLaunchKernelGGL(k_bwd_rows_dot, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, b.od,
                       b.lse, b.w, b.cq, b.wself, p.L, p.R, nt);
  else
    hipLaunchKernelGGL((k_bwd_rows<D, T>), gt, dim3(256), 0, s, b.o32, b.lse, (const T*)v,
                       (const T*)dout, b.w, b.cq, p.L, p.R, p.o_seg_rows(), nt);
  mark(2);
  if (attend_mfma_supported(p)) {
    (void)launch_backward_mfma(p, qk, v, perm, dout, knorm, b, s);
    mark(3);
    const bool half = bwd_rows_half(p);
    auto go = [&](auto r) {
      constexpr int kR = decltype(r)::value;
      if (half) {
        auto kern = k_bwd_reduce_sum<D, T, kR, _Float16>;
        hipLaunchKernelGGL(kern, gt, dim3(256), 0, s, (const T*)dout, b.wself,
                           (const _Float16*)b.dq, (const _Float16*)b.dv, (T*)dqk, (T*)dvo, p.L,
                           p.R, nt);
      } else {
        auto kern = k_bwd_reduce_sum<D, T, kR, float>;
        hipLaunchKernelGGL(kern, gt, dim3(256), 0, s, (const T*)dout, b.wself, b.dq, b.dv,
                           (T*)dqk, (T*)dvo, p.L, p.R, nt);
      }
    };
    switch (p.R) {
      case 1: go(std::integral_constant<int, 1>{}); break;
      case 2: go(std::integral_constant<int, 2>{}); break;
      case 3: go(std::integral_constant<int, 3>{}); break;
      case 4: go(std::integral_constant<int, 4>{}); break;
      case 8: go(std::integral_constant<int, 8>{}); break;
      default: go(std::integral_constant<int, 0>{}); break;
    }
    mark(4);
    return;
  }
  if (p.causal) {
    hipLaunchKernelGGL((k_bwd_dq<D, T, true>), gr, dim3(256), 0, s, (const T*)qk, (const T*)v,
                       (const T*)dout, perm, b.lse, b.w, b.cq, b.dq, p.L, p.m, p.R, nr);
    hipLaunchKernelGGL((k_bwd_dkv<D, T, true>), gr, dim3(256), 0, s, (const T*)qk, (const T*)v,
                       (const T*)dout, perm, b.lse, b.w, b.cq, b.dk, b.dv, p.L, p.m, p.R, nr);
  } else {
    hipLaunchKernelGGL((k_bwd_dq<D, T, false>), gr, dim3(256), 0, s, (const T*)qk, (const T*)v,
                       (const T*)dout, perm, b.lse, b.w, b.cq, b.dq, p.L, p.m, p.R, nr);
    hipLaunchKernelGGL((k_bwd_dkv<D, T, false>), gr, dim3(256), 0, s, (const T*)qk, (const T*)v,
                       (const T*)dout, perm, b.lse, b.w, b.cq, b.dk, b.dv, p.L, p.m, p.R, nr);
  }
  mark(3);
  hipLaunchKernelGGL((k_bwd_reduce<D, T>), gt, dim3(256), 0, s, (const T*)qk, (const T*)dout,
                     b.lse, b.w, b.dq, b.dk, b.dv, (T*)dqk, (T*)dvo, p.L, p.R, nt);
  mark(4);
}

}  // namespace

hipError_t launch_backward(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                           const void* dout, void* dqk, void* dv, float* knorm, BwdWorkspace& b,
                           hipStream_t s, const hipEvent_t* ev) {
  // the per-round attention, recomputed from the permutation in fp32
  hipError_t e;
  if (ev) (void)hipEventRecord(ev[0], s);
  if (attend_mfma_supported(p)) {
    e = launch_key_norms(p, qk, knorm, s);
    if (e == hipSuccess)
      e = launch_attend_mfma_dot(p, qk, v, perm, knorm, dout, b.od, b.lse, s);
  } else {
    e = launch_attend(p, qk, v, nullptr, nullptr, perm, nullptr, nullptr, nullptr, b.o32, b.lse,
                      s);
  }
  if (e != hipSuccess) return e;
  if (ev) (void)hipEventRecord(ev[1], s);
  const bool bf = p.dtype == LSH_ATTN_BF16;
  if (p.d == 64) {
    if (bf) launch_t<64, bf16_t>(p, qk, v, perm, dout, dqk, dv, knorm, b, s, ev);
    else launch_t<64, float>(p, qk, v, perm, dout, dqk, dv, knorm, b, s, ev);
  } else {
    if (bf) launch_t<128, bf16_t>(p, qk, v, perm, dout, dqk, dv, knorm, b, s, ev);
    else launch_t<128, float>(p, qk, v, perm, dout, dqk, dv, knorm, b, s, ev);
  }
  return hipGetLastError();
}

}  // namespace lsh
