// backward_mfma.hip -- the backward's per-round gradient products on gfx950
// matrix cores (bf16 inputs, chunk_len 64, d in {64, 128}); same definition as
// k_bwd_dq / k_bwd_dkv in backward.hip (see there for the chain rule), computed
// per chunk with v_mfma_f32_16x16x32_bf16, one kernel for dq, dkhat and dv.
//
// Operand layouts in LDS: qk and v rows row-major (one 16-byte piece per lane
// and K-step of a product over dims), and qk and dout rows by pairs of 4-row
// groups (per dim the 4 rows of group a, then of group a + 4, the layout of
// the forward's P V product), which give a product over rows its A operand.
// Per wave and 16-row block:
//   S^T  = K Q^T,  dP^T = V dO^T                 (a query block, its 128 keys)
//   dS^T = w_q P (dP - dout.out) / (sqrt(d) |k|)   -> dQ^T = K^T dS^T
//   S    = Q K^T,  dP   = dO V^T                 (a key block, the chunk's queries)
//   wP = w_q P, dS = wP (dP - dout.out)          -> dV^T += dO^T wP, dkhat^T += Q^T dS
// Rows are written at original positions, once: no atomics, deterministic.
// Two variant readings as template flags, as in the forward's kernel: NQ, unit
// queries (the logits of query i times 1/|q_i|, dkhat taking the unit query,
// and the query's own gradient, then taken with respect to the unit query,
// going through the same normalisation Jacobian as the row's unit key); SB,
// only keys in the query's bucket of the round (bucket ids staged per row).
#include "dtype.h"
#include "internal.h"
#include "rows_lds.h"
#include "walks.h"

namespace lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;

// four floats as fp16 (round to nearest even), packed in 8 bytes; values past
// the fp16 range are clamped to +-65504 (the sum over rounds counts such
// values, so the caller can tell the gradients are inaccurate)
__device__ __forceinline__ float sat16(float x) { return fminf(fmaxf(x, -65504.0f), 65504.0f); }
__device__ __forceinline__ uint2 pack_h4(float a, float b, float c, float d) {
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  const h2_t lo = {(_Float16)sat16(a), (_Float16)sat16(b)};
  const h2_t hi = {(_Float16)sat16(c), (_Float16)sat16(d)};
  return uint2{__builtin_bit_cast(uint32_t, lo), __builtin_bit_cast(uint32_t, hi)};
}
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

using rows::BLay;
using rows::load_group;
using rows::store_pair;
using rows::store_rm;
using rows::zero_lds;

// -------------------------------------------------------------------------
// Fused: one workgroup per (segment, range of consecutive chunks), 4 waves,
// walking the range one query chunk c at a time with the keys of chunks c - 1
// and c staged (slots alternate with the chunk's parity). Wave w owns query
// block w and key block w (rows 16w .. 16w + 15) of every chunk:
//   query block w of c: S^T, dP^T over the 128 keys, dS^T, dQ^T
//   key block w of c - 1 and of c: S, dP over the 64 queries of c, then
//     dV^T += dO^T (wP), dkhat^T += Q^T dS
// The keys of chunk c - 1 have then seen every query (those of c - 1 in the
// previous step, those of c now), so their rows are final: the wave holds
// dq and dkhat of the same 16 positions (the rows of block w of chunk c - 1),
// applies the key normalisation's Jacobian per round,
//   dqk_r = dq_r + (dkhat_r - khat (khat . dkhat_r)) / |k|,
// and writes dqk_r and dv_r once (at original positions, in GT: fp16 by
// default, which halves this kernel's largest output and the reduction's
// reads, or fp32 with LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS). A range's last
// step takes the queries of the chunk after it for its last keys only; the
// next range computes their dq. The next chunk's rows are loaded into
// registers at the start of each step and staged after it.
template <int D>
struct FLds {
  using L = BLay<D>;
  static constexpr int kKt = 0;                           // [2 slots][64] qk rows
  static constexpr int kVt = kKt + 2 * L::kRM;            // [2][64] v rows
  static constexpr int kKp = kVt + 2 * L::kRM;            // [2] qk rows by group pairs
  static constexpr int kDt = kKp + 2 * L::kPM;            // dout rows of the query chunk
  static constexpr int kDp = kDt + L::kRM;                // the same by group pairs
  static constexpr int kKScale = kDp + L::kPM;            // [2][64] log2(e) / (sqrt(d) |k|)
  static constexpr int kKScaleDs = kKScale + 2 * kChunk * 4;  // [2][64] 1 / (sqrt(d) |k|)
  static constexpr int kKPos = kKScaleDs + 2 * kChunk * 4;  // [2][64] original positions
  // [64] per query: lse log2(e) - log2(w), so that exp2(s - it) is w P
  static constexpr int kQLse = kKPos + 2 * kChunk * 4;
  static constexpr int kQC = kQLse + kChunk * 4;          // [64] dout . out
  static constexpr int kPn = kQC + kChunk * 4;            // [64] positions of the next chunk
  static constexpr int kBkt = kPn + kChunk * 4;           // [2][64] bucket ids (SB)
  static constexpr int kBytes = kBkt + 2 * kChunk * 4;
};

// one chunk's rows and scalars between their loads and the staging
struct FRegs {
  uint4 k[4], v[4], d[4];
  int pos, bk;
  float n2, lse, w, c;
};

// Chunks per workgroup, and workgroups in flight the grid order is shaped for.
constexpr int kFusedRange = 16;
constexpr int kFusedResident = 256;

template <int D, bool CAUSAL, typename GT, bool NQ = false, bool SB = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 1 : 2, D == 128 ? 1 : 2))) void k_bwd_fused_mfma(
    const unsigned char* __restrict__ qk, const unsigned char* __restrict__ v,
    const unsigned char* __restrict__ dout, const int32_t* __restrict__ perm,
    const float* __restrict__ knorm, const float* __restrict__ lse, const float* __restrict__ wr,
    const float* __restrict__ cq, GT* __restrict__ dqk_r, GT* __restrict__ dv_r, int L,
    int R, int nseg, int chunks_per_wg, int ranges, int group_segs,
    const uint16_t* __restrict__ buckets) {
  using Lay = BLay<D>;
  using M = FLds<D>;
  constexpr int KS = D / 32, DT = D / 16;
  extern __shared__ __align__(16) unsigned char lds[];
  const int nchunks = L / kChunk;
  // groups of group_segs segments (all rounds of a few heads), interleaved
  int64_t seg;
  int range;
  walks::range_block(blockIdx.x, group_segs, ranges, nseg, seg, range);
  const int c0 = range * chunks_per_wg;
  const int c1 = min(nchunks, c0 + chunks_per_wg);
  if (c0 >= c1) return;
  const int cend = c1 < nchunks ? c1 : c1 - 1;  // last step (c1: its queries for keys c1 - 1)
  const int64_t bh = seg / R;
  const int64_t row0 = bh * L;
  const int32_t* pm = perm + seg * L;
  const unsigned char* qkb = qk + row0 * D * 2;
  const unsigned char* vb = v + row0 * D * 2;
  const unsigned char* db = dout + row0 * D * 2;
  float* kscale = (float*)(lds + M::kKScale);
  float* kscale_ds = (float*)(lds + M::kKScaleDs);
  int* kpos = (int*)(lds + M::kKPos);
  float* qlse = (float*)(lds + M::kQLse);
  float* qc = (float*)(lds + M::kQC);
  int* pn = (int*)(lds + M::kPn);
  int* kbkt = (int*)(lds + M::kBkt);
  const int t = threadIdx.x;
  const float sc = kLog2e / sqrtf((float)D);
  const float inv_sqrt_d = 1.0f / sqrtf((float)D);
  const float sqrt_d = sqrtf((float)D);

  auto fetch = [&](FRegs& r, bool queries) {
    load_group<D>(r.k, qkb, pn);
    load_group<D>(r.v, vb, pn);
    if (queries) load_group<D>(r.d, db, pn);
    if (t < kChunk) {
      r.pos = pn[t];
      r.n2 = knorm[row0 + r.pos];
      if (SB) r.bk = buckets[seg * L + r.pos];
      if (queries) {
        r.lse = lse[seg * L + r.pos];
        r.w = wr[seg * L + r.pos];
        r.c = cq[row0 + r.pos];
      }
    }
  };
  auto stage = [&](const FRegs& r, int sl, bool queries) {
    store_rm<D>(lds + M::kKt + sl * Lay::kRM, r.k);
    store_pair<D>(lds + M::kKp + sl * Lay::kPM, r.k);
    store_rm<D>(lds + M::kVt + sl * Lay::kRM, r.v);
    if (queries) {
      store_rm<D>(lds + M::kDt, r.d);
      store_pair<D>(lds + M::kDp, r.d);
    }
    if (t < kChunk) {
      const float rn = r.n2 > 0.f ? 1.0f / sqrtf(r.n2) : 0.f;
      kscale[sl * kChunk + t] = sc * rn;
      kscale_ds[sl * kChunk + t] = rn * inv_sqrt_d;
      kpos[sl * kChunk + t] = r.pos;
      if (SB) kbkt[sl * kChunk + t] = r.bk;
      if (queries) {
        // a zero weight gives +inf here and P = 0 below
        qlse[t] = r.lse * kLog2e - __log2f(r.w);
        qc[t] = r.c;
      }
    }
  };

  FRegs r;
  if (c0 > 0) {  // the keys of chunk c0 - 1, for the dq of chunk c0
    if (t < kChunk) pn[t] = pm[(c0 - 1) * kChunk + t];
    __syncthreads();
    fetch(r, false);
    stage(r, (c0 - 1) & 1, false);
    __syncthreads();
  } else {  // chunk 0 has no previous chunk: zero keys and values in slot 1
    zero_lds(lds + M::kKt + Lay::kRM, Lay::kRM);
    zero_lds(lds + M::kVt + Lay::kRM, Lay::kRM);
    zero_lds(lds + M::kKp + Lay::kPM, Lay::kPM);
    if (t < kChunk) {
      kscale[kChunk + t] = 0.f;
      kscale_ds[kChunk + t] = 0.f;
      kpos[kChunk + t] = 0;
      kbkt[kChunk + t] = 0;
    }
  }
  if (t < kChunk) pn[t] = pm[c0 * kChunk + t];
  __syncthreads();
  fetch(r, true);
  stage(r, c0 & 1, true);
  __syncthreads();
  if (c0 + 1 <= cend && t < kChunk) pn[t] = pm[(c0 + 1) * kChunk + t];
  __syncthreads();

  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const int blk = 16 * w + lq;  // this lane's query / key row in a chunk
  floatx4_t dqa[DT], dka[DT], dva[DT];

  // key block w of slot sl against the 64 queries of slot cur: S = Q K^T and
  // dP = dO V^T per 16-query block, then dV^T and dkhat^T (unscaled) summed
  // into dka / dva over 32-query steps
  auto keys_step = [&](int sl, int cur) {
    const float ksc = kscale[sl * kChunk + blk];
    const int kp = kpos[sl * kChunk + blk];
    const int kbk = SB ? kbkt[sl * kChunk + blk] : 0;
    bf16x8_t kf[KS], vf[KS];
    {
      const unsigned char* krow = lds + M::kKt + sl * Lay::kRM + blk * Lay::kRow;
      const unsigned char* vrow = lds + M::kVt + sl * Lay::kRM + blk * Lay::kRow;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[ks] = *(const bf16x8_t*)(krow + (32 * ks + 8 * g) * 2);
        vf[ks] = *(const bf16x8_t*)(vrow + (32 * ks + 8 * g) * 2);
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      bf16x8_t wpf, dsf;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qb = 2 * e + half;
        const unsigned char* qrow = lds + M::kKt + cur * Lay::kRM + (qb * 16 + lq) * Lay::kRow;
        const unsigned char* drow = lds + M::kDt + (qb * 16 + lq) * Lay::kRow;
        floatx4_t s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *(const bf16x8_t*)(qrow + (32 * ks + 8 * g) * 2), kf[ks], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *(const bf16x8_t*)(drow + (32 * ks + 8 * g) * 2), vf[ks], dp, 0, 0, 0);
        }
        // lane holds queries qb*16 + 4g + 0..3 and this lane's key
        const int q0 = qb * 16 + 4 * g;
        const int4 qp = *(const int4*)(kpos + cur * kChunk + q0);
        const float4 ql = *(const float4*)(qlse + q0);
        const float4 qcv = *(const float4*)(qc + q0);
        const int qpv[4] = {qp.x, qp.y, qp.z, qp.w};
        const float qlv[4] = {ql.x, ql.y, ql.z, ql.w};
        const float qcc[4] = {qcv.x, qcv.y, qcv.z, qcv.w};
        float rq[4] = {1.f, 1.f, 1.f, 1.f};  // 1 / |q| (unit queries)
        int qbk[4] = {0, 0, 0, 0};
        if (NQ) {
          const float4 r4 = *(const float4*)(kscale_ds + cur * kChunk + q0);
          rq[0] = r4.x * sqrt_d, rq[1] = r4.y * sqrt_d, rq[2] = r4.z * sqrt_d, rq[3] = r4.w * sqrt_d;
        }
        if (SB) {
          const int4 b4 = *(const int4*)(kbkt + cur * kChunk + q0);
          qbk[0] = b4.x, qbk[1] = b4.y, qbk[2] = b4.z, qbk[3] = b4.w;
        }
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool masked = (CAUSAL ? kp >= qpv[b] : kp == qpv[b]) | (SB && kbk != qbk[b]);
          const float wp =
              masked ? 0.f : __builtin_amdgcn_exp2f(fmaf(NQ ? s[b] * rq[b] : s[b], ksc, -qlv[b]));
          wpf[4 * half + b] = (__bf16)wp;
          dsf[4 * half + b] = (__bf16)(wp * (dp[b] - qcc[b]) * (NQ ? rq[b] : 1.f));
        }
      }
      const int off = (g + 4 * e) * Lay::kPair + (lq >> 3) * Lay::kBlk8 + (lq & 7) * 16;
      const unsigned char* dpair = lds + M::kDp + off;
      const unsigned char* qpair = lds + M::kKp + cur * Lay::kPM + off;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dva[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8_t*)(dpair + dt * 2 * Lay::kBlk8), wpf, dva[dt], 0, 0, 0);
        dka[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8_t*)(qpair + dt * 2 * Lay::kBlk8), dsf, dka[dt], 0, 0, 0);
      }
    }
  };

  // keys_step for key block w of both slots at once (chunk c - 1 into dka /
  // dva, chunk c into dkc / dvc): the query-row operands and the pair
  // operands of the products are read once for both
  auto keys_step2 = [&](int cur, floatx4_t* dkc, floatx4_t* dvc) {
    const int prv = cur ^ 1;
    const int sls[2] = {prv, cur};
    float ksc[2];
    int kp[2], kbk[2];
    bf16x8_t kf[2][KS], vf[2][KS];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      ksc[j] = kscale[sls[j] * kChunk + blk];
      kp[j] = kpos[sls[j] * kChunk + blk];
      kbk[j] = SB ? kbkt[sls[j] * kChunk + blk] : 0;
      const unsigned char* krow = lds + M::kKt + sls[j] * Lay::kRM + blk * Lay::kRow;
      const unsigned char* vrow = lds + M::kVt + sls[j] * Lay::kRM + blk * Lay::kRow;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        kf[j][ks] = *(const bf16x8_t*)(krow + (32 * ks + 8 * g) * 2);
        vf[j][ks] = *(const bf16x8_t*)(vrow + (32 * ks + 8 * g) * 2);
      }
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      bf16x8_t wpf[2], dsf[2];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qb = 2 * e + half;
        const unsigned char* qrow = lds + M::kKt + cur * Lay::kRM + (qb * 16 + lq) * Lay::kRow;
        const unsigned char* drow = lds + M::kDt + (qb * 16 + lq) * Lay::kRow;
        bf16x8_t aq[KS], ad[KS];
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          aq[ks] = *(const bf16x8_t*)(qrow + (32 * ks + 8 * g) * 2);
          ad[ks] = *(const bf16x8_t*)(drow + (32 * ks + 8 * g) * 2);
        }
        floatx4_t sv[2], dp[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          sv[j] = floatx4_t{};
          dp[j] = floatx4_t{};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            sv[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(aq[ks], kf[j][ks], sv[j], 0, 0, 0);
            dp[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ad[ks], vf[j][ks], dp[j], 0, 0, 0);
          }
        }
        const int q0 = qb * 16 + 4 * g;
        const int4 qp = *(const int4*)(kpos + cur * kChunk + q0);
        const float4 ql = *(const float4*)(qlse + q0);
        const float4 qcv = *(const float4*)(qc + q0);
        const int qpv[4] = {qp.x, qp.y, qp.z, qp.w};
        const float qlv[4] = {ql.x, ql.y, ql.z, ql.w};
        const float qcc[4] = {qcv.x, qcv.y, qcv.z, qcv.w};
        float rq[4] = {1.f, 1.f, 1.f, 1.f};  // 1 / |q| (unit queries)
        int qbk[4] = {0, 0, 0, 0};
        if (NQ) {
          const float4 r4 = *(const float4*)(kscale_ds + cur * kChunk + q0);
          rq[0] = r4.x * sqrt_d, rq[1] = r4.y * sqrt_d, rq[2] = r4.z * sqrt_d, rq[3] = r4.w * sqrt_d;
        }
        if (SB) {
          const int4 b4 = *(const int4*)(kbkt + cur * kChunk + q0);
          qbk[0] = b4.x, qbk[1] = b4.y, qbk[2] = b4.z, qbk[3] = b4.w;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const bool masked =
                (CAUSAL ? kp[j] >= qpv[b] : kp[j] == qpv[b]) | (SB && kbk[j] != qbk[b]);
            const float wp = masked ? 0.f
                                    : __builtin_amdgcn_exp2f(fmaf(NQ ? sv[j][b] * rq[b] : sv[j][b],
                                                                  ksc[j], -qlv[b]));
            wpf[j][4 * half + b] = (__bf16)wp;
            dsf[j][4 * half + b] = (__bf16)(wp * (dp[j][b] - qcc[b]) * (NQ ? rq[b] : 1.f));
          }
      }
      const int off = (g + 4 * e) * Lay::kPair + (lq >> 3) * Lay::kBlk8 + (lq & 7) * 16;
      const unsigned char* dpair = lds + M::kDp + off;
      const unsigned char* qpair = lds + M::kKp + cur * Lay::kPM + off;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8_t a_d = *(const bf16x8_t*)(dpair + dt * 2 * Lay::kBlk8);
        const bf16x8_t a_q = *(const bf16x8_t*)(qpair + dt * 2 * Lay::kBlk8);
        dva[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_d, wpf[0], dva[dt], 0, 0, 0);
        dka[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_q, dsf[0], dka[dt], 0, 0, 0);
        dvc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_d, wpf[1], dvc[dt], 0, 0, 0);
        dkc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_q, dsf[1], dkc[dt], 0, 0, 0);
      }
    }
  };

  // dq of query block w of slot cur (chunk c) over keys of slots prv and cur
  auto query_step = [&](int c, int cur, int prv, floatx4_t* dq) {
    const int posq = kpos[cur * kChunk + blk];
    const float lse2 = qlse[blk], cqv = qc[blk];
    const float rq = NQ ? kscale_ds[cur * kChunk + blk] * sqrt_d : 1.f;  // 1 / |q|
    const int bq = SB ? kbkt[cur * kChunk + blk] : 0;
    const int kb0 = c > 0 ? 0 : 4;  // chunk 0: the first four 16-key blocks are absent
    bf16x8_t qf[KS], df[KS];
    {
      const unsigned char* qrow = lds + M::kKt + cur * Lay::kRM + blk * Lay::kRow;
      const unsigned char* drow = lds + M::kDt + blk * Lay::kRow;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[ks] = *(const bf16x8_t*)(qrow + (32 * ks + 8 * g) * 2);
        df[ks] = *(const bf16x8_t*)(drow + (32 * ks + 8 * g) * 2);
      }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) dq[dt] = floatx4_t{};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      bf16x8_t dsf;
      const int sl = e < 2 ? prv : cur;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kb = 2 * e + half;
        const unsigned char* krow = lds + M::kKt + sl * Lay::kRM + ((kb & 3) * 16 + lq) * Lay::kRow;
        const unsigned char* vrow = lds + M::kVt + sl * Lay::kRM + ((kb & 3) * 16 + lq) * Lay::kRow;
        floatx4_t s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *(const bf16x8_t*)(krow + (32 * ks + 8 * g) * 2), qf[ks], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *(const bf16x8_t*)(vrow + (32 * ks + 8 * g) * 2), df[ks], dp, 0, 0, 0);
        }
        const int key = (kb & 3) * 16 + 4 * g;
        const float4 scv4 = *(const float4*)(kscale + sl * kChunk + key);
        const float4 sdv4 = *(const float4*)(kscale_ds + sl * kChunk + key);
        const int4 kp4 = *(const int4*)(kpos + sl * kChunk + key);
        const float scv[4] = {scv4.x, scv4.y, scv4.z, scv4.w};
        const float sdv[4] = {sdv4.x, sdv4.y, sdv4.z, sdv4.w};
        const int kpv[4] = {kp4.x, kp4.y, kp4.z, kp4.w};
        int kbv[4] = {0, 0, 0, 0};
        if (SB) {
          const int4 b4 = *(const int4*)(kbkt + sl * kChunk + key);
          kbv[0] = b4.x, kbv[1] = b4.y, kbv[2] = b4.z, kbv[3] = b4.w;
        }
        const bool absent = kb < kb0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool masked =
              absent | (CAUSAL ? kpv[b] >= posq : kpv[b] == posq) | (SB && kbv[b] != bq);
          const float wp =
              masked ? 0.f : __builtin_amdgcn_exp2f(fmaf(NQ ? s[b] * rq : s[b], scv[b], -lse2));
          dsf[4 * half + b] = (__bf16)(wp * (dp[b] - cqv) * sdv[b]);
        }
      }
      const unsigned char* kp = lds + M::kKp + sl * Lay::kPM + (g + 4 * (e & 1)) * Lay::kPair +
                                (lq >> 3) * Lay::kBlk8 + (lq & 7) * 16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        dq[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8_t*)(kp + dt * 2 * Lay::kBlk8), dsf, dq[dt], 0, 0, 0);
    }
  };

  // rows 16w .. 16w + 15 of the chunk in slot sl are final: lane holds dims
  // 16 dt + 4g + 0..3 of row blk in dqa, dka, dva
  auto finish = [&](int sl) {
    const int pos = kpos[sl * kChunk + blk];
    const float rn = kscale_ds[sl * kChunk + blk] * sqrtf((float)D);  // 1 / |k|, 0 for k = 0
    const unsigned char* krow = lds + M::kKt + sl * Lay::kRM + blk * Lay::kRow + 8 * g;
    float kv[DT][4];
    float proj = 0.f;
    if (NQ) {  // the unit query's gradient joins the unit key's: both take the Jacobian
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          dka[dt][b] = fmaf(dka[dt][b], inv_sqrt_d, dqa[dt][b]) * sqrt_d;
          dqa[dt][b] = 0.f;
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const uint2 x = *(const uint2*)(krow + 32 * dt);
      kv[dt][0] = __uint_as_float(x.x << 16);
      kv[dt][1] = __uint_as_float(x.x & 0xFFFF0000u);
      kv[dt][2] = __uint_as_float(x.y << 16);
      kv[dt][3] = __uint_as_float(x.y & 0xFFFF0000u);
#pragma unroll
      for (int b = 0; b < 4; ++b) proj = fmaf(kv[dt][b], dka[dt][b], proj);
    }
    proj += __shfl_xor(proj, 16);
    proj += __shfl_xor(proj, 32);
    proj *= rn * inv_sqrt_d;  // khat . dkhat
    GT* qo = dqk_r + (seg * L + pos) * D + 4 * g;
    GT* vo = dv_r + (seg * L + pos) * D + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      float o[4];
#pragma unroll
      for (int b = 0; b < 4; ++b)
        o[b] = dqa[dt][b] + (dka[dt][b] * inv_sqrt_d - kv[dt][b] * rn * proj) * rn;
      if constexpr (sizeof(GT) == 4) {
        *(float4*)(qo + 16 * dt) = make_float4(o[0], o[1], o[2], o[3]);
        *(float4*)(vo + 16 * dt) = make_float4(dva[dt][0], dva[dt][1], dva[dt][2], dva[dt][3]);
      } else {
        *(uint2*)(qo + 16 * dt) = pack_h4(o[0], o[1], o[2], o[3]);
        *(uint2*)(vo + 16 * dt) = pack_h4(dva[dt][0], dva[dt][1], dva[dt][2], dva[dt][3]);
      }
    }
  };

  int pnext = 0;
  for (int c = c0; c <= cend; ++c) {
    const bool more = c + 1 <= cend;
    if (more) {
      fetch(r, true);
      if (c + 2 <= cend && t < kChunk) pnext = pm[(c + 2) * kChunk + t];
    }
    const int cur = c & 1, prv = cur ^ 1;
    // (at d = 64 two workgroups share a CU, and the registers of the joint
    // step would not fit their half of the file: separate steps there)
    if (D == 128 && c > c0 && c < c1) {
      // key blocks of chunks c - 1 (their last queries) and c (their first)
      floatx4_t dkc[DT], dvc[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dkc[dt] = floatx4_t{};
        dvc[dt] = floatx4_t{};
      }
      keys_step2(cur, dkc, dvc);
      finish(prv);
      query_step(c, cur, prv, dqa);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dka[dt] = dkc[dt];
        dva[dt] = dvc[dt];
      }
    } else {
      if (c > c0) {  // the last queries of the keys of chunk c - 1
        keys_step(prv, cur);
        finish(prv);
      }
      if (c < c1) {
        query_step(c, cur, prv, dqa);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dka[dt] = floatx4_t{};
          dva[dt] = floatx4_t{};
        }
        keys_step(cur, cur);
      }
    }
    __syncthreads();  // slot prv and the query chunk are no longer read
    if (more) {
      stage(r, prv, true);
      if (c + 2 <= cend && t < kChunk) pn[t] = pnext;
    }
    __syncthreads();
  }
  if (c1 == nchunks) finish((c1 - 1) & 1);  // the last chunk's keys see no later queries
}

template <int D, bool CAUSAL, typename GT, bool NQ, bool SB>
void launch_fused(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                  const void* dout, const float* knorm, const uint16_t* buckets, BwdWorkspace& b,
                  hipStream_t s) {
  const int64_t nseg = p.nseg();
  const walks::RangeShape sh =
      walks::range_shape(p.L / kChunk, nseg, p.R, kFusedRange, kFusedResident);
  auto kern = k_bwd_fused_mfma<D, CAUSAL, GT, NQ, SB>;
  hipLaunchKernelGGL(kern, dim3((unsigned)sh.blocks), dim3(kThreads), FLds<D>::kBytes, s,
                     (const unsigned char*)qk, (const unsigned char*)v,
                     (const unsigned char*)dout, perm, knorm, b.lse, b.w, b.cq, (GT*)b.dq,
                     (GT*)b.dv, p.L, p.R, (int)nseg, sh.per, sh.ranges, sh.group_segs, buckets);
}

template <int D, typename GT, bool NQ, bool SB>
void configure() {
  (void)hipFuncSetAttribute((const void*)k_bwd_fused_mfma<D, true, GT, NQ, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, FLds<D>::kBytes);
  (void)hipFuncSetAttribute((const void*)k_bwd_fused_mfma<D, false, GT, NQ, SB>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, FLds<D>::kBytes);
}

template <typename GT, bool NQ, bool SB>
void configure_all() {
  configure<64, GT, NQ, SB>();
  configure<128, GT, NQ, SB>();
}

template <typename GT, bool NQ, bool SB>
void launch_gt(const Problem& p, const void* qk, const void* v, const int32_t* perm,
               const void* dout, const float* knorm, const uint16_t* buckets, BwdWorkspace& b,
               hipStream_t s) {
  if (p.d == 64) {
    if (p.causal) launch_fused<64, true, GT, NQ, SB>(p, qk, v, perm, dout, knorm, buckets, b, s);
    else launch_fused<64, false, GT, NQ, SB>(p, qk, v, perm, dout, knorm, buckets, b, s);
  } else {
    if (p.causal) launch_fused<128, true, GT, NQ, SB>(p, qk, v, perm, dout, knorm, buckets, b, s);
    else launch_fused<128, false, GT, NQ, SB>(p, qk, v, perm, dout, knorm, buckets, b, s);
  }
}

template <typename GT>
void launch_flags(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                  const void* dout, const float* knorm, const uint16_t* buckets,
                  BwdWorkspace& b, hipStream_t s) {
  const bool nq = (p.flags & LSH_ATTN_FLAG_NORM_QUERIES) != 0;
  const bool sb = (p.flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  if (nq && sb) launch_gt<GT, true, true>(p, qk, v, perm, dout, knorm, buckets, b, s);
  else if (nq) launch_gt<GT, true, false>(p, qk, v, perm, dout, knorm, buckets, b, s);
  else if (sb) launch_gt<GT, false, true>(p, qk, v, perm, dout, knorm, buckets, b, s);
  else launch_gt<GT, false, false>(p, qk, v, perm, dout, knorm, buckets, b, s);
}

}  // namespace

hipError_t launch_backward_mfma(const Problem& p, const void* qk, const void* v,
                                const int32_t* perm, const void* dout, const float* knorm,
                                const uint16_t* buckets, BwdWorkspace& b, hipStream_t s) {
  static bool configured[kMaxDevices] = {};
  if (first_on_device(configured)) {
    configure_all<float, false, false>();
    configure_all<float, true, false>();
    configure_all<float, false, true>();
    configure_all<float, true, true>();
    configure_all<_Float16, false, false>();
    configure_all<_Float16, true, false>();
    configure_all<_Float16, false, true>();
    configure_all<_Float16, true, true>();
  }
  if (bwd_rows_half(p)) launch_flags<_Float16>(p, qk, v, perm, dout, knorm, buckets, b, s);
  else launch_flags<float>(p, qk, v, perm, dout, knorm, buckets, b, s);
  return hipGetLastError();
}

}  // namespace lsh
