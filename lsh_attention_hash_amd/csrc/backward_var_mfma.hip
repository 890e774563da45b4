// backward_var_mfma.hip -- the backward's per-round gradient products of the
// look-ahead and de-duplicated readings on gfx950 matrix cores (bf16 inputs,
// chunk_len 64, d in {64, 128}, the variant attention kernel's shapes). Same
// definition and outputs as the plain kernels k_bwd_dq_tiled and
// k_bwd_dkv_tiled in backward.hip (see there, and the chain rule beside
// k_bwd_fused_mfma): fp32 per-round rows at original positions of
//   dq_i    = sum_j dS_ij khat_j / sqrt(d)   (the unit query's with NORM_QUERIES)
//   dkhat_j = sum_i dS_ij q_i / sqrt(d)      (q_i the unit query with NORM_QUERIES)
//   dv_j    = sum_i w_r(i) P_ij dout_i,
//   dS_ij   = w_r(i) P_ij (dout_i . v_j - dout_i . out_i),
// P_ij from the recomputed logsumexp, which k_bwd_reduce then sums over the
// rounds through the key normalisation's Jacobian.
//
// One workgroup of 4 waves per (segment, chunk), 16 rows per wave:
//   k_bwd_var_dq: the chunk's queries, over the key chunks of their window
//     (the previous one, their own, and the next with LOOK_AHEAD): per 16-key
//     block S^T = K Q^T and dP^T = V dO^T, dS^T / (sqrt(d) |k|) in bf16, and
//     per 32-key step dQ^T += K^T dS^T;
//   k_bwd_var_dkv: the chunk's keys, over the query chunks whose window holds
//     them (their own, the next, and the previous with LOOK_AHEAD): per
//     16-query block S = Q K^T and dP = dO V^T, w P and dS q-scale / sqrt(d)
//     in bf16, and per 32-query step dV^T += dO^T (wP), dkhat^T += Q^T dS.
// The other side's chunk is staged in LDS, row-major for the products over
// dims and by pairs of 4-row groups for the products over rows (the layouts
// of rows_lds.h), while the next chunk's rows are loaded into registers. The
// masks are the forward's: self (and causal), the same-bucket mask, and for
// DEDUP the logit lowered by log N_ij (dedup_lanes.h).
#include <type_traits>

#include "dedup_lanes.h"
#include "dtype.h"
#include "internal.h"
#include "rows_lds.h"

namespace lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

using rows::BLay;
using rows::load_group;
using rows::store_pair;
using rows::store_rm;

constexpr int kChunk = 64;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
// the causal mask, passed with the reading's flags (a bit no public flag uses)
constexpr int kCausalFlag = 1 << 30;

__device__ __forceinline__ floatx4_t mfma(bf16x8_t a, bf16x8_t b, floatx4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// a 16 x 16 product over dims: rows 16 blk + lq of a row-major chunk (A)
// against the wave's B operands
template <int D>
__device__ __forceinline__ floatx4_t dims_product(const unsigned char* rm, int blk,
                                                  const bf16x8_t* bf) {
  using Lay = BLay<D>;
  const int lane = threadIdx.x & 63, g = lane >> 4, lq = lane & 15;
  const unsigned char* row = rm + (blk * 16 + lq) * Lay::kRow + 8 * g * 2;
  floatx4_t acc = mfma(*(const bf16x8_t*)row, bf[0], floatx4_t{});
#pragma unroll
  for (int ks = 1; ks < D / 32; ++ks) acc = mfma(*(const bf16x8_t*)(row + 64 * ks), bf[ks], acc);
  return acc;
}

// acc[dt] += (rows of a chunk by group pairs)^T times the 32-row operand
// `op`, rows 32 e .. 32 e + 31 (lane group g: rows 32 e + 4 g + 0..3 and
// 32 e + 16 + 4 g + 0..3)
template <int D>
__device__ __forceinline__ void rows_product(const unsigned char* pm, int e, bf16x8_t op,
                                             floatx4_t* acc) {
  using Lay = BLay<D>;
  const int lane = threadIdx.x & 63, g = lane >> 4, lq = lane & 15;
  const unsigned char* p = pm + (g + 4 * e) * Lay::kPair + (lq >> 3) * Lay::kBlk8 + (lq & 7) * 16;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    acc[dt] = mfma(*(const bf16x8_t*)(p + dt * 2 * Lay::kBlk8), op, acc[dt]);
}

// the wave's B operands: dims 32 ks + 8 g .. + 7 of row 16 w + lq of a
// row-major chunk
template <int D>
__device__ __forceinline__ void load_b(const unsigned char* rm, bf16x8_t* bf) {
  using Lay = BLay<D>;
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const unsigned char* row = rm + (16 * w + lq) * Lay::kRow + 8 * g * 2;
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) bf[ks] = *(const bf16x8_t*)(row + 64 * ks);
}

template <int D, bool DD>
struct QLds {
  using L = BLay<D>;
  static constexpr int kKt = 0;                          // key qk rows, row-major
  static constexpr int kVt = kKt + L::kRM;               // v rows, row-major
  static constexpr int kKp = kVt + L::kRM;               // key qk rows by group pairs
  static constexpr int kKinv = kKp + L::kPM;             // [64] 1 / (sqrt(d) |k|)
  static constexpr int kPos = kKinv + kChunk * 4;        // [64] original positions
  static constexpr int kBkt = kPos + kChunk * 4;         // [64] bucket in the round
  static constexpr int kLc = kBkt + kChunk * 4;          // [64] uint4 chunk lanes (DEDUP)
  static constexpr int kLb = kLc + (DD ? kChunk * 16 : 0);  // [64] uint4 bucket lanes
  static constexpr int kPn = kLb + (DD ? kChunk * 16 : 0);  // [64] positions to load
  static constexpr int kBytes = kPn + kChunk * 4;
};

template <int D, bool DD>
struct KLds {
  using L = BLay<D>;
  static constexpr int kQt = 0;                          // query qk rows, row-major
  static constexpr int kZt = kQt + L::kRM;               // dout rows, row-major
  static constexpr int kQp = kZt + L::kRM;               // query qk rows by group pairs
  static constexpr int kZp = kQp + L::kPM;               // dout rows by group pairs
  static constexpr int kPos = kZp + L::kPM;              // [64] original positions
  static constexpr int kL2 = kPos + kChunk * 4;          // [64] lse log2(e) (+inf: self only)
  static constexpr int kW = kL2 + kChunk * 4;            // [64] round weight
  static constexpr int kCq = kW + kChunk * 4;            // [64] dout . out
  static constexpr int kRq = kCq + kChunk * 4;           // [64] 1/|q| (1 without unit queries)
  static constexpr int kBkt = kRq + kChunk * 4;          // [64] bucket in the round
  static constexpr int kLc = kBkt + kChunk * 4;          // [64] uint4 chunk lanes (DEDUP)
  static constexpr int kLb = kLc + (DD ? kChunk * 16 : 0);  // [64] uint4 bucket lanes
  static constexpr int kPn = kLb + (DD ? kChunk * 16 : 0);  // [64] positions to load
  static constexpr int kBytes = kPn + kChunk * 4;
};

// one chunk's rows and per-row data between their loads and the staging
struct Rows {
  uint4 a[4], b[4];
  int pos, bk;
  float n2, l, w, c;
  uint32_t lc[dedup::kMaxRounds / 2], lb[dedup::kMaxRounds / 2];
};

// -------------------------------------------------------------------------
// dq of the queries of chunk c (wave w: queries 16 w + lq)
template <int D, bool DD>
__global__ __launch_bounds__(kThreads) void k_bwd_var_dq(
    const unsigned char* __restrict__ qk, const unsigned char* __restrict__ v,
    const unsigned char* __restrict__ dout, const int32_t* __restrict__ perm,
    const float* __restrict__ knorm, const float* __restrict__ lse, const float* __restrict__ wr,
    const float* __restrict__ cq, const uint16_t* __restrict__ bkt,
    const int32_t* __restrict__ inv, float* __restrict__ dq, int L, int R, int flags) {
  using M = QLds<D, DD>;
  constexpr int KS = D / 32, DT = D / 16;
  extern __shared__ __align__(16) unsigned char lds[];
  const int nchunks = L / kChunk;
  const int64_t seg = blockIdx.x / (unsigned)nchunks;
  const int c = (int)(blockIdx.x - seg * nchunks);
  const int64_t bh = seg / R, row0 = bh * L;
  const int32_t* pm = perm + seg * L;
  const unsigned char* qkb = qk + row0 * D * 2;
  const unsigned char* vb = v + row0 * D * 2;
  const bool causal = (flags & kCausalFlag) != 0;
  const bool la = (flags & LSH_ATTN_FLAG_LOOK_AHEAD) != 0;
  const bool sb = (flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  const bool nq = (flags & LSH_ATTN_FLAG_NORM_QUERIES) != 0;
  const int32_t* inv_bh = DD ? inv + bh * R * L : nullptr;  // inv is read only with DEDUP
  const uint16_t* bk_bh = bkt + bh * R * L;
  float* kinv = (float*)(lds + M::kKinv);
  int* kpos = (int*)(lds + M::kPos);
  int* kbk = (int*)(lds + M::kBkt);
  uint4* klc = (uint4*)(lds + M::kLc);
  uint4* klb = (uint4*)(lds + M::kLb);
  int* pn = (int*)(lds + M::kPn);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const float rsd = 1.0f / sqrtf((float)D);

  // the chunk's query and dout rows, as the waves' B operands
  if (t < kChunk) pn[t] = pm[c * kChunk + t];
  __syncthreads();
  {
    uint4 a[4], z[4];
    load_group<D>(a, qkb, pn);
    load_group<D>(z, dout + row0 * D * 2, pn);
    store_rm<D>(lds + M::kKt, a);
    store_rm<D>(lds + M::kVt, z);
  }
  __syncthreads();
  bf16x8_t qf[KS], zf[KS];
  load_b<D>(lds + M::kKt, qf);
  load_b<D>(lds + M::kVt, zf);
  const int q = 16 * w + lq;
  const int posq = pn[q];
  const float l = lse[seg * L + posq];
  const bool live = l != kSelfLogit;  // a query that saw only itself has dq = 0
  const float l2 = l * kLog2e, wq = wr[seg * L + posq], cqv = cq[row0 + posq];
  float rq = 1.0f;
  if (nq) {
    const float n2 = knorm[row0 + posq];
    rq = n2 > 0.f ? 1.0f / sqrtf(n2) : 0.f;
  }
  const int bq = sb ? bkt[seg * L + posq] : 0;
  uint32_t qc[4] = {0u, 0u, 0u, 0u}, qb[4] = {0u, 0u, 0u, 0u};
  if (DD) {
    uint32_t kc[4];
    dedup::row_lanes(inv_bh, bk_bh, R, L, kChunk, posq, sb, kc, qb);
    dedup::query_lanes(kc, R, qc);
  }

  auto fetch = [&](Rows& r) {
    load_group<D>(r.a, qkb, pn);
    load_group<D>(r.b, vb, pn);
    if (t < kChunk) {
      r.pos = pn[t];
      r.n2 = knorm[row0 + r.pos];
      if (sb) r.bk = bkt[seg * L + r.pos];
      if (DD) dedup::row_lanes(inv_bh, bk_bh, R, L, kChunk, r.pos, sb, r.lc, r.lb);
    }
  };
  auto stage = [&](const Rows& r) {
    store_rm<D>(lds + M::kKt, r.a);
    store_rm<D>(lds + M::kVt, r.b);
    store_pair<D>(lds + M::kKp, r.a);
    if (t < kChunk) {
      kinv[t] = r.n2 > 0.f ? rsd / sqrtf(r.n2) : 0.f;
      kpos[t] = r.pos;
      if (sb) kbk[t] = r.bk;
      if (DD) {
        klc[t] = make_uint4(r.lc[0], r.lc[1], r.lc[2], r.lc[3]);
        klb[t] = make_uint4(r.lb[0], r.lb[1], r.lb[2], r.lb[3]);
      }
    }
  };

  floatx4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = floatx4_t{};
  const int x0 = c > 0 ? c - 1 : c;
  const int x1 = la && c + 1 < nchunks ? c + 1 : c;
  __syncthreads();  // every wave holds its operands: the row area is free
  if (t < kChunk) pn[t] = pm[x0 * kChunk + t];
  __syncthreads();
  Rows r;
  fetch(r);
  for (int x = x0; x <= x1; ++x) {
    stage(r);
    if (x < x1 && t < kChunk) pn[t] = pm[(x + 1) * kChunk + t];
    __syncthreads();
    if (x < x1) fetch(r);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      bf16x8_t op;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kb = 2 * e + half;
        const floatx4_t s = dims_product<D>(lds + M::kKt, kb, qf);
        const floatx4_t dp = dims_product<D>(lds + M::kVt, kb, zf);
        const int key = 16 * kb + 4 * g;
        const float4 ki = *(const float4*)(kinv + key);
        const int4 kp = *(const int4*)(kpos + key);
        int4 kbv = {0, 0, 0, 0};
        if (sb) kbv = *(const int4*)(kbk + key);
        const float kis[4] = {ki.x, ki.y, ki.z, ki.w};
        const int kps[4] = {kp.x, kp.y, kp.z, kp.w}, kbs[4] = {kbv.x, kbv.y, kbv.z, kbv.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool masked = !live || (causal ? kps[b] >= posq : kps[b] == posq) ||
                              (sb && kbs[b] != bq);
          float x2 = fmaf(s[b], kis[b] * rq * kLog2e, -l2);
          if (DD) {
            const uint4 c4 = klc[key + b], b4 = klb[key + b];
            const uint32_t kc[4] = {c4.x, c4.y, c4.z, c4.w}, kbw[4] = {b4.x, b4.y, b4.z, b4.w};
            x2 -= dedup::log2_rounds(qc, qb, kc, kbw, R, la, sb);
          }
          const float p = masked ? 0.f : __builtin_amdgcn_exp2f(x2);
          op[4 * half + b] = (__bf16)(wq * p * (dp[b] - cqv) * kis[b]);
        }
      }
      rows_product<D>(lds + M::kKp, e, op, acc);
    }
    __syncthreads();  // every wave is done with the staged chunk
  }
  float* drow = dq + (seg * L + posq) * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *(float4*)(drow + 16 * dt) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
}

// -------------------------------------------------------------------------
// dkhat and dv of the keys of chunk c (wave w: keys 16 w + lq); SB: the
// same-bucket mask (a template flag here: its per-query bucket lanes are what
// the de-duplicated form at d = 128 cannot fit). Two workgroups per CU (75 KB
// of LDS each at d = 128) where the registers allow it without spills: all
// but the de-duplicated form with the same-bucket mask at d = 128.
template <int D, bool DD, bool SB>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(DD && SB && D == 128 ? 1 : 2,
                                   DD && SB && D == 128 ? 1 : 2))) void k_bwd_var_dkv(
    const unsigned char* __restrict__ qk, const unsigned char* __restrict__ v,
    const unsigned char* __restrict__ dout, const int32_t* __restrict__ perm,
    const float* __restrict__ knorm, const float* __restrict__ lse, const float* __restrict__ wr,
    const float* __restrict__ cq, const uint16_t* __restrict__ bkt,
    const int32_t* __restrict__ inv, float* __restrict__ dk, float* __restrict__ dv, int L,
    int R, int flags) {
  using M = KLds<D, DD>;
  constexpr int KS = D / 32, DT = D / 16;
  extern __shared__ __align__(16) unsigned char lds[];
  const int nchunks = L / kChunk;
  const int64_t seg = blockIdx.x / (unsigned)nchunks;
  const int c = (int)(blockIdx.x - seg * nchunks);
  const int64_t bh = seg / R, row0 = bh * L;
  const int32_t* pm = perm + seg * L;
  const unsigned char* qkb = qk + row0 * D * 2;
  const unsigned char* zb = dout + row0 * D * 2;
  const bool causal = (flags & kCausalFlag) != 0;
  const bool la = (flags & LSH_ATTN_FLAG_LOOK_AHEAD) != 0;
  constexpr bool sb = SB;
  const bool nq = (flags & LSH_ATTN_FLAG_NORM_QUERIES) != 0;
  const int32_t* inv_bh = DD ? inv + bh * R * L : nullptr;  // inv is read only with DEDUP
  const uint16_t* bk_bh = bkt + bh * R * L;
  int* qpos = (int*)(lds + M::kPos);
  float* ql2 = (float*)(lds + M::kL2);
  float* qw = (float*)(lds + M::kW);
  float* qcq = (float*)(lds + M::kCq);
  float* qrq = (float*)(lds + M::kRq);
  int* qbk = (int*)(lds + M::kBkt);
  uint4* qlc = (uint4*)(lds + M::kLc);
  uint4* qlb = (uint4*)(lds + M::kLb);
  int* pn = (int*)(lds + M::kPn);
  const int t = threadIdx.x, lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const float rsd = 1.0f / sqrtf((float)D);

  // the chunk's key and value rows, as the waves' B operands
  if (t < kChunk) pn[t] = pm[c * kChunk + t];
  __syncthreads();
  {
    uint4 a[4], b[4];
    load_group<D>(a, qkb, pn);
    load_group<D>(b, v + row0 * D * 2, pn);
    store_rm<D>(lds + M::kQt, a);
    store_rm<D>(lds + M::kZt, b);
  }
  __syncthreads();
  bf16x8_t kf[KS], vf[KS];
  load_b<D>(lds + M::kQt, kf);
  load_b<D>(lds + M::kZt, vf);
  const int posk = pn[16 * w + lq];
  const float kn2 = knorm[row0 + posk];
  const float kinv = kn2 > 0.f ? 1.0f / sqrtf(kn2) : 0.f;  // 1/|k|
  const int bkk = sb ? bkt[seg * L + posk] : 0;
  uint32_t kc[4] = {0u, 0u, 0u, 0u}, kbw[4] = {0u, 0u, 0u, 0u};
  if (DD) dedup::row_lanes(inv_bh, bk_bh, R, L, kChunk, posk, sb, kc, kbw);

  auto fetch = [&](Rows& r) {
    load_group<D>(r.a, qkb, pn);
    load_group<D>(r.b, zb, pn);
    if (t < kChunk) {
      r.pos = pn[t];
      r.l = lse[seg * L + r.pos];
      r.w = wr[seg * L + r.pos];
      r.c = cq[row0 + r.pos];
      if (nq) r.n2 = knorm[row0 + r.pos];
      if (sb) r.bk = bkt[seg * L + r.pos];
      if (DD) dedup::row_lanes(inv_bh, bk_bh, R, L, kChunk, r.pos, sb, r.lc, r.lb);
    }
  };
  auto stage = [&](const Rows& r) {
    store_rm<D>(lds + M::kQt, r.a);
    store_rm<D>(lds + M::kZt, r.b);
    store_pair<D>(lds + M::kQp, r.a);
    store_pair<D>(lds + M::kZp, r.b);
    if (t < kChunk) {
      qpos[t] = r.pos;
      ql2[t] = r.l == kSelfLogit ? INFINITY : r.l * kLog2e;  // self only: no pair
      qw[t] = r.w;
      qcq[t] = r.c;
      qrq[t] = nq ? (r.n2 > 0.f ? 1.0f / sqrtf(r.n2) : 0.f) : 1.0f;
      if (sb) qbk[t] = r.bk;
      if (DD) {
        uint32_t qc[4];
        dedup::query_lanes(r.lc, R, qc);
        qlc[t] = make_uint4(qc[0], qc[1], qc[2], qc[3]);
        qlb[t] = make_uint4(r.lb[0], r.lb[1], r.lb[2], r.lb[3]);
      }
    }
  };

  floatx4_t ak[DT], av[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) ak[dt] = av[dt] = floatx4_t{};
  // the query chunks whose window holds chunk c
  const int y0 = la && c > 0 ? c - 1 : c;
  const int y1 = c + 1 < nchunks ? c + 1 : c;
  __syncthreads();  // every wave holds its operands: the row area is free
  if (t < kChunk) pn[t] = pm[y0 * kChunk + t];
  __syncthreads();
  Rows r;
  fetch(r);
  for (int y = y0; y <= y1; ++y) {
    stage(r);
    if (y < y1 && t < kChunk) pn[t] = pm[(y + 1) * kChunk + t];
    __syncthreads();
    if (y < y1) fetch(r);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      bf16x8_t opv, opk;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qb = 2 * e + half;
        const floatx4_t s = dims_product<D>(lds + M::kQt, qb, kf);
        const floatx4_t dp = dims_product<D>(lds + M::kZt, qb, vf);
        const int qi = 16 * qb + 4 * g;
        const int4 qp = *(const int4*)(qpos + qi);
        const float4 l4 = *(const float4*)(ql2 + qi), w4 = *(const float4*)(qw + qi);
        const float4 c4 = *(const float4*)(qcq + qi), r4 = *(const float4*)(qrq + qi);
        int4 b4 = {0, 0, 0, 0};
        if (sb) b4 = *(const int4*)(qbk + qi);
        const int qps[4] = {qp.x, qp.y, qp.z, qp.w}, qbs[4] = {b4.x, b4.y, b4.z, b4.w};
        const float l2s[4] = {l4.x, l4.y, l4.z, l4.w}, ws[4] = {w4.x, w4.y, w4.z, w4.w};
        const float cs[4] = {c4.x, c4.y, c4.z, c4.w}, rs[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool masked = (causal ? posk >= qps[b] : posk == qps[b]) || (sb && qbs[b] != bkk);
          float x2 = fmaf(s[b], kinv * rsd * rs[b] * kLog2e, -l2s[b]);
          if (DD) {
            const uint4 lc4 = qlc[qi + b], lb4 = qlb[qi + b];
            const uint32_t qc[4] = {lc4.x, lc4.y, lc4.z, lc4.w};
            const uint32_t qbw[4] = {lb4.x, lb4.y, lb4.z, lb4.w};
            x2 -= dedup::log2_rounds(qc, qbw, kc, kbw, R, la, sb);
          }
          const float p = masked ? 0.f : __builtin_amdgcn_exp2f(x2);
          const float wp = ws[b] * p;
          opv[4 * half + b] = (__bf16)wp;
          opk[4 * half + b] = (__bf16)(wp * (dp[b] - cs[b]) * rs[b] * rsd);
        }
      }
      rows_product<D>(lds + M::kZp, e, opv, av);
      rows_product<D>(lds + M::kQp, e, opk, ak);
    }
    __syncthreads();  // every wave is done with the staged chunk
  }
  float* krow = dk + (seg * L + posk) * D + 4 * g;
  float* vrow = dv + (seg * L + posk) * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    *(float4*)(krow + 16 * dt) = make_float4(ak[dt][0], ak[dt][1], ak[dt][2], ak[dt][3]);
    *(float4*)(vrow + 16 * dt) = make_float4(av[dt][0], av[dt][1], av[dt][2], av[dt][3]);
  }
}

template <int D, bool DD, bool SB>
void launch_dd(const Problem& p, const void* qk, const void* v, const int32_t* perm,
               const void* dout, const float* knorm, const uint16_t* bkt, const int32_t* inv,
               BwdWorkspace& b, hipStream_t s) {
  constexpr int qbytes = QLds<D, DD>::kBytes, kbytes = KLds<D, DD>::kBytes;
  static bool configured[kMaxDevices] = {};
  if (first_on_device(configured)) {
    (void)hipFuncSetAttribute((const void*)k_bwd_var_dq<D, DD>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, qbytes);
    (void)hipFuncSetAttribute((const void*)k_bwd_var_dkv<D, DD, SB>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, kbytes);
  }
  const dim3 grid((unsigned)(p.nseg() * (p.L / kChunk)));
  const int flags = (p.flags & kVariantFlags) | (p.causal ? kCausalFlag : 0);
  hipLaunchKernelGGL((k_bwd_var_dq<D, DD>), grid, dim3(kThreads), qbytes, s,
                     (const unsigned char*)qk, (const unsigned char*)v,
                     (const unsigned char*)dout, perm, knorm, b.lse, b.w, b.cq, bkt, inv, b.dq,
                     p.L, p.R, flags);
  hipLaunchKernelGGL((k_bwd_var_dkv<D, DD, SB>), grid, dim3(kThreads), kbytes, s,
                     (const unsigned char*)qk, (const unsigned char*)v,
                     (const unsigned char*)dout, perm, knorm, b.lse, b.w, b.cq, bkt, inv, b.dk,
                     b.dv, p.L, p.R, flags);
}

}  // namespace

hipError_t launch_backward_var_mfma(const Problem& p, const void* qk, const void* v,
                                    const int32_t* perm, const void* dout, const float* knorm,
                                    const uint16_t* buckets, const int32_t* inv,
                                    BwdWorkspace& b, hipStream_t s) {
  const bool dd = (p.flags & LSH_ATTN_FLAG_DEDUP) != 0;
  const bool sb = (p.flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  auto go = [&](auto dv_, auto ddv, auto sbv) {
    launch_dd<decltype(dv_)::value, decltype(ddv)::value, decltype(sbv)::value>(
        p, qk, v, perm, dout, knorm, buckets, inv, b, s);
  };
  using T = std::true_type;
  using F = std::false_type;
  using D64 = std::integral_constant<int, 64>;
  using D128 = std::integral_constant<int, 128>;
  if (p.d == 64) {
    if (dd) sb ? go(D64{}, T{}, T{}) : go(D64{}, T{}, F{});
    else sb ? go(D64{}, F{}, T{}) : go(D64{}, F{}, F{});
  } else {
    if (dd) sb ? go(D128{}, T{}, T{}) : go(D128{}, T{}, F{});
    else sb ? go(D128{}, F{}, T{}) : go(D128{}, F{}, F{});
  }
  return hipGetLastError();
}

}  // namespace lsh
