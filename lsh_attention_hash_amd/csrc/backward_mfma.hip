// backward_mfma.hip -- the backward's dq and (dkhat, dv) products on gfx950
// matrix cores (bf16 inputs, chunk_len 64, d in {64, 128}); same definition and
// outputs as k_bwd_dq / k_bwd_dkv in backward.hip (see there for the chain
// rule), computed per chunk with v_mfma_f32_16x16x32_bf16.
//
// dq: one workgroup per (segment, query chunk c), 4 waves x 16 queries. The
//   window (chunks c-1 and c) is staged in LDS: qk rows row-major (Kt) and by
//   pairs of 4-key groups (Kp: per dim the 4 keys of group a then of group
//   a + 4, as the forward stages v), v rows row-major (Vt). Per wave:
//     S^T  = K Q^T       (A = Kt rows, B = the queries' rows)
//     dP^T = V dO^T      (A = Vt rows, B = the queries' dout rows)
//     dS^T = w_q P (dP - dout.out) / (sqrt(d) |k|)    (registers)
//     dQ^T = K^T dS^T    (A = Kp, B = dS^T of two 16-key blocks, in the
//                         key order of the forward's P V product)
// dkv: one workgroup per (segment, key chunk c), 4 waves x 16 keys; the
//   queries that see the chunk are those of chunks c and c + 1, staged one
//   chunk at a time (qk and dout rows, row-major and by pairs of groups).
//   Per wave and 16-query block:
//     S  = Q K^T, dP = dO V^T   (A = query rows, B = the wave's key rows)
//     wP = w_q P, dS = wP (dP - dout.out)
//   then over 32-query steps:
//     dV^T    += dO^T (wP)      (A = dout by pairs of query groups)
//     dkhat^T += Q^T dS / sqrt(d)
// Rows are written at original positions, once: no atomics, deterministic.
#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BLay {
  static constexpr int kSegs = D / 8;               // 16-byte pieces per row
  static constexpr int kRow = D * 2 + 16;           // row-major stride (bytes, +16 pad)
  static constexpr int kBlk8 = 8 * 16 + 16;         // 8 dims of a group pair (+16 pad)
  static constexpr int kPair = D / 8 * kBlk8;       // one pair of 4-row groups
  static constexpr int kRM = kChunk * kRow;         // a chunk, row-major
  static constexpr int kPM = kChunk / 8 * kPair;    // a chunk, by group pairs
  static constexpr int kUsers = (kChunk / 4) * kSegs;  // (group, piece) loaders
  static_assert(kUsers <= kThreads, "one group piece per thread");
};

// Thread t < kUsers loads piece t % kSegs of the 4 rows of group t / kSegs
// (rows at the positions pn[] of a chunk, from rows of `D` bf16 at `base`).
template <int D>
__device__ __forceinline__ void load_group(uint4* r, const unsigned char* base, const int* pn) {
  using Lay = BLay<D>;
  const int t = threadIdx.x;
  if (t < Lay::kUsers) {
    const int qd = t / Lay::kSegs, sg = t % Lay::kSegs;
    const int4 p4 = *(const int4*)(pn + 4 * qd);
    const int pos[4] = {p4.x, p4.y, p4.z, p4.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = *(const uint4*)(base + (int64_t)pos[k] * (D * 2) + sg * 16);
  }
}

// the same registers, row-major
template <int D>
__device__ __forceinline__ void store_rm(unsigned char* dst, const uint4* r) {
  using Lay = BLay<D>;
  const int t = threadIdx.x;
  if (t < Lay::kUsers) {
    const int qd = t / Lay::kSegs, sg = t % Lay::kSegs;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      uint4 x = r[k];
      asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
      *(uint4*)(dst + (4 * qd + k) * Lay::kRow + sg * 16) = x;
    }
  }
}

// the same registers by group pairs: group qd is half (qd / 4) % 2 of pair
// (qd % 4) + 4 (qd / 8); per dim 8 bytes of its 4 rows
template <int D>
__device__ __forceinline__ void store_pair(unsigned char* dst, const uint4* r) {
  using Lay = BLay<D>;
  const int t = threadIdx.x;
  if (t < Lay::kUsers) {
    const int qd = t / Lay::kSegs, sg = t % Lay::kSegs;
    const int pair = (qd & 3) + 4 * (qd >> 3), half = (qd >> 2) & 1;
    unsigned char* d = dst + pair * Lay::kPair + sg * Lay::kBlk8 + half * 8;
    const uint32_t w0[4] = {r[0].x, r[0].y, r[0].z, r[0].w};
    const uint32_t w1[4] = {r[1].x, r[1].y, r[1].z, r[1].w};
    const uint32_t w2[4] = {r[2].x, r[2].y, r[2].z, r[2].w};
    const uint32_t w3[4] = {r[3].x, r[3].y, r[3].z, r[3].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *(uint2*)(d + 32 * u) =
          make_uint2((w0[u] & 0xFFFFu) | (w1[u] << 16), (w2[u] & 0xFFFFu) | (w3[u] << 16));
      *(uint2*)(d + 32 * u + 16) = make_uint2((w0[u] >> 16) | (w1[u] & 0xFFFF0000u),
                                              (w2[u] >> 16) | (w3[u] & 0xFFFF0000u));
    }
  }
}

__device__ __forceinline__ void zero_lds(unsigned char* p, int bytes) {
  for (int i = threadIdx.x; i < bytes / 16; i += kThreads) ((uint4*)p)[i] = uint4{};
}

// -------------------------------------------------------------------------
template <int D>
struct DqLds {
  using L = BLay<D>;
  static constexpr int kKt = 0;                         // [2][64 rows]
  static constexpr int kVt = kKt + 2 * L::kRM;
  static constexpr int kKp = kVt + 2 * L::kRM;          // [2][8 pairs]
  static constexpr int kScale = kKp + 2 * L::kPM;       // [2][64] log2(e) / (sqrt(d) |k|)
  static constexpr int kPos = kScale + 2 * kChunk * 4;  // [2][64]
  static constexpr int kBytes = kPos + 2 * kChunk * 4;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void k_bwd_dq_mfma(
    const unsigned char* __restrict__ qk, const unsigned char* __restrict__ v,
    const unsigned char* __restrict__ dout, const int32_t* __restrict__ perm,
    const float* __restrict__ knorm, const float* __restrict__ lse, const float* __restrict__ wr,
    const float* __restrict__ cq, float* __restrict__ dq, int L, int R) {
  using Lay = BLay<D>;
  using M = DqLds<D>;
  constexpr int KS = D / 32, DT = D / 16;
  extern __shared__ __align__(16) unsigned char lds[];
  const int nchunks = L / kChunk;
  const int64_t seg = blockIdx.x / (unsigned)nchunks;
  const int c = (int)(blockIdx.x - seg * nchunks);
  const int64_t bh = seg / R;
  const int64_t row0 = bh * L;
  const int32_t* pm = perm + seg * L;
  const unsigned char* qkb = qk + row0 * D * 2;
  const unsigned char* vb = v + row0 * D * 2;
  int* pn = (int*)(lds + M::kPos);  // positions (slot 0: chunk c - 1, slot 1: chunk c)
  float* kscale = (float*)(lds + M::kScale);
  const int t = threadIdx.x;
  if (t < kChunk) pn[kChunk + t] = pm[c * kChunk + t];
  else if (t < 2 * kChunk) pn[t - kChunk] = c > 0 ? pm[(c - 1) * kChunk + t - kChunk] : 0;
  __syncthreads();
  {
    uint4 kr[2][4], vr[2][4];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      load_group<D>(kr[sl], qkb, pn + sl * kChunk);
      load_group<D>(vr[sl], vb, pn + sl * kChunk);
    }
    float n2 = 0.f;
    if (t < 2 * kChunk) n2 = knorm[row0 + pn[t]];
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      if (sl == 0 && c == 0) continue;
      store_rm<D>(lds + M::kKt + sl * Lay::kRM, kr[sl]);
      store_pair<D>(lds + M::kKp + sl * Lay::kPM, kr[sl]);
      store_rm<D>(lds + M::kVt + sl * Lay::kRM, vr[sl]);
    }
    if (t < 2 * kChunk) {
      const float sc = kLog2e / sqrtf((float)D);
      kscale[t] = (n2 > 0.f && (t >= kChunk || c > 0)) ? sc / sqrtf(n2) : 0.f;
    }
    if (c == 0) {  // no previous chunk: zero keys and values in slot 0
      zero_lds(lds + M::kKt, Lay::kRM);
      zero_lds(lds + M::kVt, Lay::kRM);
      zero_lds(lds + M::kKp, Lay::kPM);
    }
  }
  __syncthreads();

  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const int q = 16 * w + lq;
  const int posq = pn[kChunk + q];
  const int64_t sq = seg * L + posq;
  const float lse2 = lse[sq] * kLog2e;
  const float wq = wr[sq], cqv = cq[row0 + posq];
  const int kb0 = c > 0 ? 0 : 4;  // chunk 0: the first four 16-key blocks are absent
  bf16x8_t qf[KS], df[KS];
  {
    const unsigned char* qrow = lds + M::kKt + (kChunk + q) * Lay::kRow;
    const unsigned char* drow = dout + (row0 + posq) * D * 2;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = *(const bf16x8_t*)(qrow + (32 * ks + 8 * g) * 2);
      df[ks] = *(const bf16x8_t*)(drow + (32 * ks + 8 * g) * 2);
    }
  }
  floatx4_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = floatx4_t{};
  const float inv_log2e = 1.0f / kLog2e;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bf16x8_t dsf;
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int kb = 2 * e + half;
      const int sl = kb < 4 ? 0 : 1;
      const unsigned char* krow = lds + M::kKt + sl * Lay::kRM + ((kb & 3) * 16 + lq) * Lay::kRow;
      const unsigned char* vrow = lds + M::kVt + sl * Lay::kRM + ((kb & 3) * 16 + lq) * Lay::kRow;
      floatx4_t s = {}, dp = {};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)(krow + (32 * ks + 8 * g) * 2),
                                                     qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)(vrow + (32 * ks + 8 * g) * 2),
                                                      df[ks], dp, 0, 0, 0);
      }
      const int key = (kb & 3) * 16 + 4 * g;
      const float4 sc = *(const float4*)(kscale + sl * kChunk + key);
      const int4 kp = *(const int4*)(pn + sl * kChunk + key);
      const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
      const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
      const bool absent = kb < kb0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        const bool masked = absent | (CAUSAL ? kpv[b] >= posq : kpv[b] == posq);
        const float p = masked ? 0.f : __builtin_amdgcn_exp2f(fmaf(s[b], scv[b], -lse2));
        dsf[4 * half + b] = (__bf16)(wq * p * (dp[b] - cqv) * scv[b] * inv_log2e);
      }
    }
    const int sl = e < 2 ? 0 : 1;
    const unsigned char* kp = lds + M::kKp + sl * Lay::kPM + (g + 4 * (e & 1)) * Lay::kPair +
                              (lq >> 3) * Lay::kBlk8 + (lq & 7) * 16;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
          *(const bf16x8_t*)(kp + dt * 2 * Lay::kBlk8), dsf, acc[dt], 0, 0, 0);
  }
  // lane holds dims 16 dt + 4g + 0..3 of query q
  float* orow = dq + sq * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    *(float4*)(orow + 16 * dt) = make_float4(acc[dt][0], acc[dt][1], acc[dt][2], acc[dt][3]);
}

// -------------------------------------------------------------------------
template <int D>
struct DkvLds {
  using L = BLay<D>;
  static constexpr int kKt = 0;                       // keys of chunk c
  static constexpr int kVt = kKt + L::kRM;
  static constexpr int kQt = kVt + L::kRM;            // queries of the staged chunk
  static constexpr int kDt = kQt + L::kRM;            // their dout rows
  static constexpr int kQp = kDt + L::kRM;
  static constexpr int kDp = kQp + L::kPM;
  static constexpr int kKScale = kDp + L::kPM;        // [64]
  static constexpr int kKPos = kKScale + kChunk * 4;  // [64]
  static constexpr int kQPos = kKPos + kChunk * 4;    // [64]
  static constexpr int kQLse = kQPos + kChunk * 4;    // [64] lse * log2(e)
  static constexpr int kQW = kQLse + kChunk * 4;      // [64] round weight
  static constexpr int kQC = kQW + kChunk * 4;        // [64] dout . out
  static constexpr int kBytes = kQC + kChunk * 4;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void k_bwd_dkv_mfma(
    const unsigned char* __restrict__ qk, const unsigned char* __restrict__ v,
    const unsigned char* __restrict__ dout, const int32_t* __restrict__ perm,
    const float* __restrict__ knorm, const float* __restrict__ lse, const float* __restrict__ wr,
    const float* __restrict__ cq, float* __restrict__ dk, float* __restrict__ dv, int L, int R) {
  using Lay = BLay<D>;
  using M = DkvLds<D>;
  constexpr int KS = D / 32, DT = D / 16;
  extern __shared__ __align__(16) unsigned char lds[];
  const int nchunks = L / kChunk;
  const int64_t seg = blockIdx.x / (unsigned)nchunks;
  const int c = (int)(blockIdx.x - seg * nchunks);
  const int64_t bh = seg / R;
  const int64_t row0 = bh * L;
  const int32_t* pm = perm + seg * L;
  const unsigned char* qkb = qk + row0 * D * 2;
  const unsigned char* vb = v + row0 * D * 2;
  const unsigned char* db = dout + row0 * D * 2;
  float* kscale = (float*)(lds + M::kKScale);
  int* kpos = (int*)(lds + M::kKPos);
  int* qpos = (int*)(lds + M::kQPos);
  float* qlse = (float*)(lds + M::kQLse);
  float* qw = (float*)(lds + M::kQW);
  float* qc = (float*)(lds + M::kQC);
  const int t = threadIdx.x;
  // the keys: chunk c
  if (t < kChunk) kpos[t] = pm[c * kChunk + t];
  __syncthreads();
  {
    uint4 kr[4], vr[4];
    load_group<D>(kr, qkb, kpos);
    load_group<D>(vr, vb, kpos);
    float n2 = 0.f;
    if (t < kChunk) n2 = knorm[row0 + kpos[t]];
    store_rm<D>(lds + M::kKt, kr);
    store_rm<D>(lds + M::kVt, vr);
    if (t < kChunk) kscale[t] = n2 > 0.f ? kLog2e / sqrtf((float)D) / sqrtf(n2) : 0.f;
  }
  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const int key = 16 * w + lq;  // this lane's key (B operand column) in the chunk
  floatx4_t dka[DT], dva[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dka[dt] = floatx4_t{};
    dva[dt] = floatx4_t{};
  }
  for (int h = 0; h < 2; ++h) {
    const int cq_idx = c + h;
    if (cq_idx >= nchunks) break;
    __syncthreads();  // the previous query chunk is no longer read
    if (t < kChunk) qpos[t] = pm[cq_idx * kChunk + t];
    __syncthreads();
    {
      uint4 qr[4], dr[4];
      load_group<D>(qr, qkb, qpos);
      load_group<D>(dr, db, qpos);
      float l = 0.f, wv = 0.f, cv = 0.f;
      if (t < kChunk) {
        const int64_t sq = seg * L + qpos[t];
        l = lse[sq];
        wv = wr[sq];
        cv = cq[row0 + qpos[t]];
      }
      store_rm<D>(lds + M::kQt, qr);
      store_pair<D>(lds + M::kQp, qr);
      store_rm<D>(lds + M::kDt, dr);
      store_pair<D>(lds + M::kDp, dr);
      if (t < kChunk) {
        qlse[t] = l * kLog2e;
        qw[t] = wv;
        qc[t] = cv;
      }
    }
    __syncthreads();
    const float ksc = kscale[key];
    const int kp = kpos[key];
    const unsigned char* krow = lds + M::kKt + key * Lay::kRow;
    const unsigned char* vrow = lds + M::kVt + key * Lay::kRow;
    bf16x8_t kf[KS], vf[KS];
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      kf[ks] = *(const bf16x8_t*)(krow + (32 * ks + 8 * g) * 2);
      vf[ks] = *(const bf16x8_t*)(vrow + (32 * ks + 8 * g) * 2);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      bf16x8_t wpf, dsf;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int qb = 2 * e + half;
        const unsigned char* qrow = lds + M::kQt + (qb * 16 + lq) * Lay::kRow;
        const unsigned char* drow = lds + M::kDt + (qb * 16 + lq) * Lay::kRow;
        floatx4_t s = {}, dp = {};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(*(const bf16x8_t*)(qrow + (32 * ks + 8 * g) * 2),
                                                       kf[ks], s, 0, 0, 0);
          dp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              *(const bf16x8_t*)(drow + (32 * ks + 8 * g) * 2), vf[ks], dp, 0, 0, 0);
        }
        // lane holds queries qb*16 + 4g + 0..3 and this lane's key
        const int q0 = qb * 16 + 4 * g;
        const int4 qp = *(const int4*)(qpos + q0);
        const float4 ql = *(const float4*)(qlse + q0);
        const float4 qwv = *(const float4*)(qw + q0);
        const float4 qcv = *(const float4*)(qc + q0);
        const int qpv[4] = {qp.x, qp.y, qp.z, qp.w};
        const float qlv[4] = {ql.x, ql.y, ql.z, ql.w};
        const float qww[4] = {qwv.x, qwv.y, qwv.z, qwv.w};
        const float qcc[4] = {qcv.x, qcv.y, qcv.z, qcv.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const bool masked = CAUSAL ? kp >= qpv[b] : kp == qpv[b];
          const float p = masked ? 0.f : __builtin_amdgcn_exp2f(fmaf(s[b], ksc, -qlv[b]));
          const float wp = qww[b] * p;
          wpf[4 * half + b] = (__bf16)wp;
          dsf[4 * half + b] = (__bf16)(wp * (dp[b] - qcc[b]));
        }
      }
      const int off = (g + 4 * e) * Lay::kPair + (lq >> 3) * Lay::kBlk8 + (lq & 7) * 16;
      const unsigned char* dpair = lds + M::kDp + off;
      const unsigned char* qpair = lds + M::kQp + off;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        dva[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8_t*)(dpair + dt * 2 * Lay::kBlk8), wpf, dva[dt], 0, 0, 0);
        dka[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8_t*)(qpair + dt * 2 * Lay::kBlk8), dsf, dka[dt], 0, 0, 0);
      }
    }
  }
  // lane holds dims 16 dt + 4g + 0..3 of this lane's key
  const float scale = 1.0f / sqrtf((float)D);
  const int64_t sk = seg * L + kpos[key];
  float* krow_o = dk + sk * D + 4 * g;
  float* vrow_o = dv + sk * D + 4 * g;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    *(float4*)(krow_o + 16 * dt) = make_float4(dka[dt][0] * scale, dka[dt][1] * scale,
                                               dka[dt][2] * scale, dka[dt][3] * scale);
    *(float4*)(vrow_o + 16 * dt) = make_float4(dva[dt][0], dva[dt][1], dva[dt][2], dva[dt][3]);
  }
}

template <int D, bool CAUSAL>
void launch_d(const Problem& p, const void* qk, const void* v, const int32_t* perm,
              const void* dout, const float* knorm, BwdWorkspace& b, hipStream_t s,
              hipEvent_t after_dq) {
  const dim3 grid((unsigned)(p.nseg() * (p.L / kChunk)));
  hipLaunchKernelGGL((k_bwd_dq_mfma<D, CAUSAL>), grid, dim3(kThreads), DqLds<D>::kBytes, s,
                     (const unsigned char*)qk, (const unsigned char*)v,
                     (const unsigned char*)dout, perm, knorm, b.lse, b.w, b.cq, b.dq, p.L, p.R);
  if (after_dq) (void)hipEventRecord(after_dq, s);
  hipLaunchKernelGGL((k_bwd_dkv_mfma<D, CAUSAL>), grid, dim3(kThreads), DkvLds<D>::kBytes, s,
                     (const unsigned char*)qk, (const unsigned char*)v,
                     (const unsigned char*)dout, perm, knorm, b.lse, b.w, b.cq, b.dk, b.dv, p.L,
                     p.R);
}

template <int D>
void configure() {
  (void)hipFuncSetAttribute((const void*)k_bwd_dq_mfma<D, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, DqLds<D>::kBytes);
  (void)hipFuncSetAttribute((const void*)k_bwd_dq_mfma<D, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, DqLds<D>::kBytes);
  (void)hipFuncSetAttribute((const void*)k_bwd_dkv_mfma<D, true>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, DkvLds<D>::kBytes);
  (void)hipFuncSetAttribute((const void*)k_bwd_dkv_mfma<D, false>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, DkvLds<D>::kBytes);
}

}  // namespace

hipError_t launch_backward_mfma(const Problem& p, const void* qk, const void* v,
                                const int32_t* perm, const void* dout, const float* knorm,
                                BwdWorkspace& b, hipStream_t s, hipEvent_t after_dq) {
  static bool configured = false;
  if (!configured) {
    configure<64>();
    configure<128>();
    configured = true;
  }
  if (p.d == 64) {
    if (p.causal) launch_d<64, true>(p, qk, v, perm, dout, knorm, b, s, after_dq);
    else launch_d<64, false>(p, qk, v, perm, dout, knorm, b, s, after_dq);
  } else {
    if (p.causal) launch_d<128, true>(p, qk, v, perm, dout, knorm, b, s, after_dq);
    else launch_d<128, false>(p, qk, v, perm, dout, knorm, b, s, after_dq);
  }
  return hipGetLastError();
}

}  // namespace lsh
