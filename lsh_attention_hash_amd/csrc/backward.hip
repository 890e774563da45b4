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
// On the matrix-core path (bf16, chunk_len 64, d in {64, 128}, the default
// reading) the dq and (dkhat, dv) products run in one kernel of
// backward_mfma.hip instead of the two below; it also applies the
// normalisation per round, so its reduction (k_bwd_reduce_sum) only sums.
// The variant readings take the plain kernels below: the window and the
// logits are those of the forward's reading (the overview, section 2.1:
// look-ahead chunk, same-bucket mask, unit queries; de-duplicated rounds,
// www.2kiu.com/news/5253576/, section 2.2: P divided by the number of rounds
// sharing the pair), and with unit queries q / |q| the query's gradient is
// taken with respect to the unit query, which goes through the same
// normalisation Jacobian as the row's unit key.
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

// DEDUP: the number of rounds whose window holds key j for query i (the self
// and causal masks do not depend on the round); inv_bh, bk_bh: [R, L] of one
// (b, h), bk_bh read with SAME_BUCKET.
__device__ __forceinline__ int shared_rounds(const int32_t* inv_bh, const uint16_t* bk_bh, int L,
                                             int m, int R, int i, int j, int flags) {
  int n = 0;
  for (int r = 0; r < R; ++r) {
    const int64_t o = (int64_t)r * L;
    const int ci = inv_bh[o + i] / m, cj = inv_bh[o + j] / m;
    bool in = cj == ci || cj == ci - 1 || ((flags & LSH_ATTN_FLAG_LOOK_AHEAD) && cj == ci + 1);
    if ((flags & LSH_ATTN_FLAG_SAME_BUCKET) && bk_bh[o + j] != bk_bh[o + i]) in = false;
    n += in;
  }
  return n;
}

// The plain gradient products (any shape, every variant reading), in the
// plain attention kernel's layout: a workgroup of 256 threads takes kQB
// queries (k_bwd_dq_tiled: dq = sum over the window of dS_ij khat_j / sqrt(d))
// or kQB keys (k_bwd_dkv_tiled: dkhat_j = sum_i dS_ij q_i / sqrt(d) and
// dv_j = sum_i w_r(i) P_ij dout_i over the queries that see the key: those of
// its chunk and of the next one, and of the previous one with LOOK_AHEAD) of
// one chunk, 16 threads per row. The other side's rows are staged in LDS as
// fp32, kKB at a time, the next block loaded into registers while the current
// one is used. A thread computes the pairs of its row with the staged rows
// g + 16 u (full dot products from LDS), writes the pair coefficients to LDS,
// and then accumulates its kDPT output dims over the block. The variant
// readings change the window and the logits as in the forward: LOOK_AHEAD adds
// the next chunk, SAME_BUCKET drops keys of other buckets (bkt [seg, L]),
// NORM_QUERIES takes the unit query (and dq is then the gradient with respect
// to it), DEDUP lowers each logit by log of the number of rounds sharing the
// pair (inv [seg, L]).
template <int D>
struct BT {
  static constexpr int kQB = 16;                     // rows per workgroup
  static constexpr int kKB = D == 64 ? 64 : 32;      // staged rows per block
  static constexpr int kPPT = kKB / 16;              // pairs per thread per block
  static constexpr int kDPT = D / 16;                // output dims per thread
  static constexpr int kS = D + 4;                   // LDS row stride (fp32 words)
  static constexpr int kPieces = kKB * D / 4 / 256;  // 4-element loads per thread per array
  static constexpr int kTPR = 256 / kKB;             // threads per staged row in norm passes
  static constexpr int kMaxWin = 3 * 256;            // window slots (chunk_len <= 256)
};

__device__ __forceinline__ float4 load4f(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 load4f(const bf16_t* p) {
  const uint2 u = *(const uint2*)p;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

template <int D>
__device__ __forceinline__ float lds_dot(const float* a, const float* b) {
  float s = 0.f;
#pragma unroll
  for (int col = 0; col < D; col += 4) {
    const float4 x = *(const float4*)(a + col);
    const float4 y = *(const float4*)(b + col);
    s = fmaf(x.x, y.x, s);
    s = fmaf(x.y, y.y, s);
    s = fmaf(x.z, y.z, s);
    s = fmaf(x.w, y.w, s);
  }
  return s;
}

template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(256) void k_bwd_dq_tiled(
    const T* __restrict__ qk, const T* __restrict__ v, const T* __restrict__ dout,
    const int32_t* __restrict__ perm, const float* __restrict__ lse, const float* __restrict__ w,
    const float* __restrict__ cq, float* __restrict__ dq, int L, int m, int R, int flags,
    const uint16_t* __restrict__ bkt, const int32_t* __restrict__ inv) {
  using S = BT<D>;
  __shared__ __align__(16) float ks[S::kKB * S::kS];
  __shared__ __align__(16) float vs[S::kKB * S::kS];
  __shared__ __align__(16) float qs[S::kQB * S::kS];
  __shared__ __align__(16) float zs[S::kQB * S::kS];
  __shared__ float cs[S::kQB * S::kKB];
  __shared__ float nrm[S::kKB];
  __shared__ int pw[S::kMaxWin];
  __shared__ uint16_t bw[S::kMaxWin];
  const int tid = threadIdx.x;
  const int qblocks = (m + S::kQB - 1) / S::kQB;
  const int nchunks = L / m;
  const int64_t seg = blockIdx.x / (unsigned)(nchunks * qblocks);
  const int rest = (int)(blockIdx.x - seg * (nchunks * qblocks));
  const int c = rest / qblocks, qb = rest % qblocks;
  const int64_t bh = seg / R;
  const int32_t* pm = perm + seg * L;
  const bool sb = (flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  const bool dedup = (flags & LSH_ATTN_FLAG_DEDUP) != 0;
  const int first = (c > 0 ? c - 1 : c) * m;
  int last = (c + 1) * m;
  if ((flags & LSH_ATTN_FLAG_LOOK_AHEAD) && last < L) last += m;
  const int nwin = last - first;
  for (int x = tid; x < nwin; x += 256) {
    const int j = pm[first + x];
    pw[x] = j;
    if (sb) bw[x] = bkt[seg * L + j];
  }
  __syncthreads();
  const int q = tid / 16, g = tid % 16;
  const int qslot0 = c * m + qb * S::kQB;
  const int nq = min(S::kQB, (c + 1) * m - qslot0);
  for (int p = tid; p < S::kQB * D / 4; p += 256) {
    const int ql = p / (D / 4), col = (p % (D / 4)) * 4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), z = a;
    if (ql < nq) {
      const int64_t row = (bh * L + pw[qslot0 + ql - first]) * D + col;
      a = load4f(qk + row);
      z = load4f(dout + row);
    }
    *(float4*)&qs[ql * S::kS + col] = a;
    *(float4*)&zs[ql * S::kS + col] = z;
  }
  const bool active = q < nq;
  const int i = active ? pw[qslot0 + q - first] : 0;
  const int bi = sb && active ? bw[qslot0 + q - first] : 0;
  const float l = active ? lse[seg * L + i] : kSelfLogit;
  const bool live = active && l != kSelfLogit;  // a self-only query has dq = 0
  const float wi = live ? w[seg * L + i] : 0.f, ci = live ? cq[bh * L + i] : 0.f;
  __syncthreads();
  if (flags & LSH_ATTN_FLAG_NORM_QUERIES) {  // the unit query, as the forward takes it
    float qq = 0.f;
#pragma unroll
    for (int u = 0; u < S::kDPT; ++u) {
      const float x = qs[q * S::kS + g * S::kDPT + u];
      qq += x * x;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) qq += __shfl_xor(qq, off);
    const float rq = qq > 0.f ? 1.0f / sqrtf(qq) : 0.f;
#pragma unroll
    for (int u = 0; u < S::kDPT; ++u) qs[q * S::kS + g * S::kDPT + u] *= rq;
    __syncthreads();
  }
  float4 kr[S::kPieces], vr[S::kPieces];
  auto fetch = [&](int kb) {
    const int t0 = kb * S::kKB;
#pragma unroll
    for (int u = 0; u < S::kPieces; ++u) {
      const int p = tid + 256 * u;
      const int kk = p / (D / 4), col = (p % (D / 4)) * 4;
      const int x = t0 + kk;
      if (x < nwin) {
        const int64_t row = (bh * L + pw[x]) * D + col;
        kr[u] = load4f(qk + row);
        vr[u] = load4f(v + row);
      } else {
        kr[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        vr[u] = kr[u];
      }
    }
  };
  const float scale = 1.0f / sqrtf((float)D);
  float acc[S::kDPT];
#pragma unroll
  for (int u = 0; u < S::kDPT; ++u) acc[u] = 0.f;
  const int nblk = (nwin + S::kKB - 1) / S::kKB;
  fetch(0);
  for (int kb = 0; kb < nblk; ++kb) {
    const int t0 = kb * S::kKB;
    const int nk = min(S::kKB, nwin - t0);
#pragma unroll
    for (int u = 0; u < S::kPieces; ++u) {
      const int p = tid + 256 * u;
      const int kk = p / (D / 4), col = (p % (D / 4)) * 4;
      *(float4*)&ks[kk * S::kS + col] = kr[u];
      *(float4*)&vs[kk * S::kS + col] = vr[u];
    }
    if (kb + 1 < nblk) fetch(kb + 1);
    __syncthreads();
    {  // squared key norms, as the forward sums them
      const int kk = tid / S::kTPR, part = tid % S::kTPR;
      float nn = 0.f;
#pragma unroll
      for (int u = 0; u < D / S::kTPR; ++u) {
        const float x = ks[kk * S::kS + part * (D / S::kTPR) + u];
        nn += x * x;
      }
#pragma unroll
      for (int off = 1; off < S::kTPR; off <<= 1) nn += __shfl_xor(nn, off);
      if (part == 0) nrm[kk] = nn;
    }
    __syncthreads();
#pragma unroll
    for (int u = 0; u < S::kPPT; ++u) {
      const int kk = g + 16 * u;
      float cv = 0.f;
      if (live && kk < nk) {
        const int j = pw[t0 + kk];
        const bool keep = j != i && !(CAUSAL && j > i) && !(sb && bw[t0 + kk] != bi);
        if (keep) {
          const float nn = nrm[kk];
          const float rn = nn > 0.f ? 1.0f / sqrtf(nn) : 0.f;
          float logit = nn > 0.f ? lds_dot<D>(qs + q * S::kS, ks + kk * S::kS) / sqrtf(nn) * scale
                                 : 0.f;
          if (dedup) logit -= __logf((float)shared_rounds(inv + bh * R * L, bkt + bh * R * L, L,
                                                          m, R, i, j, flags));
          const float p = __expf(logit - l);
          const float dvd = lds_dot<D>(zs + q * S::kS, vs + kk * S::kS);
          cv = wi * p * (dvd - ci) * rn * scale;
        }
      }
      cs[q * S::kKB + kk] = cv;
    }
    // the 16 threads of a query (one wave) wrote its coefficients; each reads them all
    for (int kk = 0; kk < nk; ++kk) {
      const float cv = cs[q * S::kKB + kk];
#pragma unroll
      for (int u = 0; u < S::kDPT; u += 4) {
        const float4 b = *(const float4*)&ks[kk * S::kS + g * S::kDPT + u];
        acc[u] = fmaf(cv, b.x, acc[u]);
        acc[u + 1] = fmaf(cv, b.y, acc[u + 1]);
        acc[u + 2] = fmaf(cv, b.z, acc[u + 2]);
        acc[u + 3] = fmaf(cv, b.w, acc[u + 3]);
      }
    }
    __syncthreads();
  }
  if (!active) return;
  float* drow = dq + (seg * L + i) * D + g * S::kDPT;
#pragma unroll
  for (int u = 0; u < S::kDPT; u += 4)
    *(float4*)(drow + u) = make_float4(acc[u], acc[u + 1], acc[u + 2], acc[u + 3]);
}

template <int D, typename T, bool CAUSAL>
__global__ __launch_bounds__(256) void k_bwd_dkv_tiled(
    const T* __restrict__ qk, const T* __restrict__ v, const T* __restrict__ dout,
    const int32_t* __restrict__ perm, const float* __restrict__ lse, const float* __restrict__ w,
    const float* __restrict__ cq, float* __restrict__ dk, float* __restrict__ dv, int L, int m,
    int R, int flags, const uint16_t* __restrict__ bkt, const int32_t* __restrict__ inv) {
  using S = BT<D>;
  __shared__ __align__(16) float ks[S::kQB * S::kS];
  __shared__ __align__(16) float vs[S::kQB * S::kS];
  __shared__ __align__(16) float qs[S::kKB * S::kS];
  __shared__ __align__(16) float zs[S::kKB * S::kS];
  __shared__ float ca[S::kQB * S::kKB];
  __shared__ float cb[S::kQB * S::kKB];
  __shared__ float qsc[S::kKB];
  __shared__ int pw[S::kMaxWin];
  __shared__ uint16_t bw[S::kMaxWin];
  const int tid = threadIdx.x;
  const int kblocks = (m + S::kQB - 1) / S::kQB;
  const int nchunks = L / m;
  const int64_t seg = blockIdx.x / (unsigned)(nchunks * kblocks);
  const int rest = (int)(blockIdx.x - seg * (nchunks * kblocks));
  const int c = rest / kblocks, kbk = rest % kblocks;
  const int64_t bh = seg / R;
  const int32_t* pm = perm + seg * L;
  const bool sb = (flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  const bool dedup = (flags & LSH_ATTN_FLAG_DEDUP) != 0;
  const bool nqf = (flags & LSH_ATTN_FLAG_NORM_QUERIES) != 0;
  // the queries that see the keys of chunk c: chunks c and c + 1, and c - 1
  // with the look-ahead window
  const int first = ((flags & LSH_ATTN_FLAG_LOOK_AHEAD) && c > 0 ? c - 1 : c) * m;
  const int last = min(L, (c + 2) * m);
  const int nwin = last - first;
  for (int x = tid; x < nwin; x += 256) {
    const int i = pm[first + x];
    pw[x] = i;
    if (sb) bw[x] = bkt[seg * L + i];
  }
  const int key = tid / 16, g = tid % 16;
  const int kslot0 = c * m + kbk * S::kQB;
  const int nk = min(S::kQB, (c + 1) * m - kslot0);
  for (int p = tid; p < S::kQB * D / 4; p += 256) {
    const int kl = p / (D / 4), col = (p % (D / 4)) * 4;
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
    if (kl < nk) {
      const int64_t row = (bh * L + pm[kslot0 + kl]) * D + col;
      a = load4f(qk + row);
      b = load4f(v + row);
    }
    *(float4*)&ks[kl * S::kS + col] = a;
    *(float4*)&vs[kl * S::kS + col] = b;
  }
  const bool active = key < nk;
  const int j = active ? pm[kslot0 + key] : 0;
  const int bj = sb && active ? bkt[seg * L + j] : 0;
  __syncthreads();
  float kn = 0.f;  // |k_j|^2 over the 16 threads of the key
#pragma unroll
  for (int u = 0; u < S::kDPT; ++u) {
    const float x = ks[key * S::kS + g * S::kDPT + u];
    kn += x * x;
  }
#pragma unroll
  for (int off = 1; off < 16; off <<= 1) kn += __shfl_xor(kn, off);
  const float rn = kn > 0.f ? 1.0f / sqrtf(kn) : 0.f;
  float4 qr[S::kPieces], zr[S::kPieces];
  auto fetch = [&](int qb) {
    const int s0 = qb * S::kKB;
#pragma unroll
    for (int u = 0; u < S::kPieces; ++u) {
      const int p = tid + 256 * u;
      const int qq = p / (D / 4), col = (p % (D / 4)) * 4;
      const int x = s0 + qq;
      if (x < nwin) {
        const int64_t row = (bh * L + pw[x]) * D + col;
        qr[u] = load4f(qk + row);
        zr[u] = load4f(dout + row);
      } else {
        qr[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        zr[u] = qr[u];
      }
    }
  };
  const float scale = 1.0f / sqrtf((float)D);
  float gk[S::kDPT], gv[S::kDPT];
#pragma unroll
  for (int u = 0; u < S::kDPT; ++u) {
    gk[u] = 0.f;
    gv[u] = 0.f;
  }
  const int nblk = (nwin + S::kKB - 1) / S::kKB;
  fetch(0);
  for (int qb = 0; qb < nblk; ++qb) {
    const int s0 = qb * S::kKB;
    const int nqb = min(S::kKB, nwin - s0);
#pragma unroll
    for (int u = 0; u < S::kPieces; ++u) {
      const int p = tid + 256 * u;
      const int qq = p / (D / 4), col = (p % (D / 4)) * 4;
      *(float4*)&qs[qq * S::kS + col] = qr[u];
      *(float4*)&zs[qq * S::kS + col] = zr[u];
    }
    if (qb + 1 < nblk) fetch(qb + 1);
    __syncthreads();
    if (nqf) {  // unit queries: kTPR threads per staged query
      const int qq = tid / S::kTPR, part = tid % S::kTPR;
      float nn = 0.f;
#pragma unroll
      for (int u = 0; u < D / S::kTPR; ++u) {
        const float x = qs[qq * S::kS + part * (D / S::kTPR) + u];
        nn += x * x;
      }
#pragma unroll
      for (int off = 1; off < S::kTPR; off <<= 1) nn += __shfl_xor(nn, off);
      if (part == 0) qsc[qq] = nn > 0.f ? 1.0f / sqrtf(nn) : 0.f;
      __syncthreads();
    }
#pragma unroll
    for (int u = 0; u < S::kPPT; ++u) {
      const int qq = g + 16 * u;
      float a = 0.f, b = 0.f;
      if (active && qq < nqb) {
        const int i = pw[s0 + qq];
        bool keep = i != j && !(CAUSAL && j > i) && !(sb && bw[s0 + qq] != bj);
        const float l = keep ? lse[seg * L + i] : kSelfLogit;
        if (keep && l != kSelfLogit) {
          const float qs_i = nqf ? qsc[qq] : 1.f;
          float logit = lds_dot<D>(qs + qq * S::kS, ks + key * S::kS) * qs_i * rn * scale;
          if (dedup) logit -= __logf((float)shared_rounds(inv + bh * R * L, bkt + bh * R * L, L,
                                                          m, R, i, j, flags));
          const float p = __expf(logit - l);
          const float dvd = lds_dot<D>(zs + qq * S::kS, vs + key * S::kS);
          const float wi = w[seg * L + i], ci = cq[bh * L + i];
          a = wi * p * (dvd - ci) * scale * qs_i;
          b = wi * p;
        }
      }
      ca[key * S::kKB + qq] = a;
      cb[key * S::kKB + qq] = b;
    }
    // the 16 threads of a key (one wave) wrote its coefficients; each reads them all
    for (int qq = 0; qq < nqb; ++qq) {
      const float a = ca[key * S::kKB + qq], b = cb[key * S::kKB + qq];
#pragma unroll
      for (int u = 0; u < S::kDPT; u += 4) {
        const float4 x = *(const float4*)&qs[qq * S::kS + g * S::kDPT + u];
        const float4 z = *(const float4*)&zs[qq * S::kS + g * S::kDPT + u];
        gk[u] = fmaf(a, x.x, gk[u]);
        gk[u + 1] = fmaf(a, x.y, gk[u + 1]);
        gk[u + 2] = fmaf(a, x.z, gk[u + 2]);
        gk[u + 3] = fmaf(a, x.w, gk[u + 3]);
        gv[u] = fmaf(b, z.x, gv[u]);
        gv[u + 1] = fmaf(b, z.y, gv[u + 1]);
        gv[u + 2] = fmaf(b, z.z, gv[u + 2]);
        gv[u + 3] = fmaf(b, z.w, gv[u + 3]);
      }
    }
    __syncthreads();
  }
  if (!active) return;
  float* krow = dk + (seg * L + j) * D + g * S::kDPT;
  float* vrow = dv + (seg * L + j) * D + g * S::kDPT;
#pragma unroll
  for (int u = 0; u < S::kDPT; u += 4) {
    *(float4*)(krow + u) = make_float4(gk[u], gk[u + 1], gk[u + 2], gk[u + 3]);
    *(float4*)(vrow + u) = make_float4(gv[u], gv[u + 1], gv[u + 2], gv[u + 3]);
  }
}

// the forward's int32 bucket ids as the kernels' u16 ids
__global__ void k_bwd_bucket16(const int32_t* __restrict__ b32, uint16_t* __restrict__ b16,
                               int64_t n) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x < n) b16[x] = (uint16_t)b32[x];
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
                                                    int L, int R, int64_t n_rows, bool nq) {
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
  if (nq) {  // dq is then the gradient of the unit query: it shares the key's Jacobian
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      gk[u] += gq[u];
      gq[u] = 0.f;
    }
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
                                                        int L, int R_rt, int64_t n_rows,
                                                        unsigned long long* __restrict__ at_limit) {
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
  uint32_t lim = 0;
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
      // fp16 rows clamped at +-65504 by the product kernel: a half-word whose
      // magnitude bits reach 0x7BFF carries into its sign bit here
      typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const u32x4_t ba = __builtin_bit_cast(u32x4_t, a[u]);
        const u32x4_t bc = __builtin_bit_cast(u32x4_t, c[u]);
#pragma unroll
        for (int k = 0; k < 4; ++k)
          lim |= ((ba[k] & 0x7FFF7FFFu) + 0x04010401u) | ((bc[k] & 0x7FFF7FFFu) + 0x04010401u);
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
  if (lim & 0x80008000u) atomicAdd(at_limit, 1ull);
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
              const void* dout, void* dqk, void* dvo, const float* knorm, const uint16_t* bk16,
              const int32_t* inv, BwdWorkspace& b, unsigned long long* at_limit, hipStream_t s,
              const hipEvent_t* ev) {
  auto mark = [&](int j) {
    if (ev) (void)hipEventRecord(ev[j], s);
  };
  const int64_t rpb = 256 / (D / 8);
  const int64_t nt = p.n_token_heads(), nr = p.n_rows();
  const dim3 gt((unsigned)((nt + rpb - 1) / rpb)), gr((unsigned)((nr + rpb - 1) / rpb));
  if (bwd_recompute_dot(p))
    hipLaunchKernelGGL(k_bwd_rows_dot, dim3((unsigned)((nt + 255) / 256)), dim3(256), 0, s, b.od,
                       b.lse, b.w, b.cq, b.wself, p.L, p.R, nt);
  else
    hipLaunchKernelGGL((k_bwd_rows<D, T>), gt, dim3(256), 0, s, b.o32, b.lse, (const T*)v,
                       (const T*)dout, b.w, b.cq, p.L, p.R, p.o_seg_rows(), nt);
  mark(2);
  if (bwd_mfma_supported(p)) {
    (void)launch_backward_mfma(p, qk, v, perm, dout, knorm, bk16, b, s);
    mark(3);
    const bool half = bwd_rows_half(p);
    auto go = [&](auto r) {
      constexpr int kR = decltype(r)::value;
      if (half) {
        auto kern = k_bwd_reduce_sum<D, T, kR, _Float16>;
        hipLaunchKernelGGL(kern, gt, dim3(256), 0, s, (const T*)dout, b.wself,
                           (const _Float16*)b.dq, (const _Float16*)b.dv, (T*)dqk, (T*)dvo, p.L,
                           p.R, nt, at_limit);
      } else {
        auto kern = k_bwd_reduce_sum<D, T, kR, float>;
        hipLaunchKernelGGL(kern, gt, dim3(256), 0, s, (const T*)dout, b.wself, b.dq, b.dv,
                           (T*)dqk, (T*)dvo, p.L, p.R, nt, at_limit);
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
  const int vf = p.flags & kVariantFlags;
  const dim3 gq((unsigned)(p.nseg() * (p.L / p.m) * ((p.m + BT<D>::kQB - 1) / BT<D>::kQB)));
  if (bwd_recompute_dot(p)) {  // look-ahead, de-duplication: products on matrix cores
    (void)launch_backward_var_mfma(p, qk, v, perm, dout, knorm, bk16, inv, b, s);
  } else if (p.causal) {
    hipLaunchKernelGGL((k_bwd_dq_tiled<D, T, true>), gq, dim3(256), 0, s, (const T*)qk,
                       (const T*)v, (const T*)dout, perm, b.lse, b.w, b.cq, b.dq, p.L, p.m, p.R,
                       vf, bk16, inv);
    hipLaunchKernelGGL((k_bwd_dkv_tiled<D, T, true>), gq, dim3(256), 0, s, (const T*)qk,
                       (const T*)v, (const T*)dout, perm, b.lse, b.w, b.cq, b.dk, b.dv, p.L, p.m,
                       p.R, vf, bk16, inv);
  } else {
    hipLaunchKernelGGL((k_bwd_dq_tiled<D, T, false>), gq, dim3(256), 0, s, (const T*)qk,
                       (const T*)v, (const T*)dout, perm, b.lse, b.w, b.cq, b.dq, p.L, p.m, p.R,
                       vf, bk16, inv);
    hipLaunchKernelGGL((k_bwd_dkv_tiled<D, T, false>), gq, dim3(256), 0, s, (const T*)qk,
                       (const T*)v, (const T*)dout, perm, b.lse, b.w, b.cq, b.dk, b.dv, p.L, p.m,
                       p.R, vf, bk16, inv);
  }
  mark(3);
  hipLaunchKernelGGL((k_bwd_reduce<D, T>), gt, dim3(256), 0, s, (const T*)qk, (const T*)dout,
                     b.lse, b.w, b.dq, b.dk, b.dv, (T*)dqk, (T*)dvo, p.L, p.R, nt,
                     (p.flags & LSH_ATTN_FLAG_NORM_QUERIES) != 0);
  mark(4);
}

}  // namespace

hipError_t launch_backward(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                           const int32_t* buckets, const void* dout, void* dqk, void* dv,
                           float* knorm, uint16_t* bk16, int32_t* inv, BwdWorkspace& b,
                           unsigned long long* at_limit, hipStream_t s, const hipEvent_t* ev) {
  // the per-round attention, recomputed from the permutation
  hipError_t e = hipSuccess;
  if (ev) (void)hipEventRecord(ev[0], s);
  if (p.flags & LSH_ATTN_FLAG_SAME_BUCKET) {
    const int64_t n = p.n_rows();
    hipLaunchKernelGGL(k_bwd_bucket16, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s,
                       buckets, bk16, n);
  }
  if (p.flags & LSH_ATTN_FLAG_DEDUP) e = launch_inverse_perm(p, perm, inv, s);
  if (e != hipSuccess) return e;
  if (bwd_mfma_supported(p)) {
    e = launch_key_norms(p, qk, knorm, s);
    if (e == hipSuccess)
      e = launch_attend_mfma_dot(p, qk, v, perm, knorm, dout, bk16, b.od, b.lse, s);
  } else if (bwd_recompute_dot(p)) {
    // look-ahead, de-duplication: the variant kernel reduced to dout . o_r
    e = launch_key_norms(p, qk, knorm, s);
    if (e == hipSuccess)
      e = launch_attend_variant_dot(p, qk, v, perm, knorm, dout, bk16, inv, b.od, b.lse, s);
  } else {
    // fp32 rows from the plain kernel, which takes every variant reading
    e = launch_attend_plain(p, qk, v, perm, bk16, inv, b.o32, b.lse, s);
  }
  if (e != hipSuccess) return e;
  if (ev) (void)hipEventRecord(ev[1], s);
  const bool bf = p.dtype == LSH_ATTN_BF16;
  if (p.d == 64) {
    if (bf) launch_t<64, bf16_t>(p, qk, v, perm, dout, dqk, dv, knorm, bk16, inv, b, at_limit, s, ev);
    else launch_t<64, float>(p, qk, v, perm, dout, dqk, dv, knorm, bk16, inv, b, at_limit, s, ev);
  } else {
    if (bf) launch_t<128, bf16_t>(p, qk, v, perm, dout, dqk, dv, knorm, bk16, inv, b, at_limit, s, ev);
    else launch_t<128, float>(p, qk, v, perm, dout, dqk, dv, knorm, bk16, inv, b, at_limit, s, ev);
  }
  return hipGetLastError();
}

}  // namespace lsh
