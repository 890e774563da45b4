// attend_variants.hip -- the chunk attention of the variant readings on gfx950
// matrix cores (bf16 inputs, chunk_len 64, d in {64, 128}).
//
// The readings (flags; the definition is the plain kernel's in attend.hip):
//   LOOK_AHEAD   the window is the previous, the current and the next chunk
//                (Reformer overview, www.dtcms.com/a/488796.html, section 2.1:
//                one neighbouring group before and one after);
//   SAME_BUCKET  only keys in the query's bucket of the round (same page, the
//                mask M of its attention formula);
//   NORM_QUERIES queries unit-normalised too (same page, section 2.1);
//   DEDUP        a key that several rounds give a query counts once
//                (www.2kiu.com/news/5253576/, section 2.2): each logit is
//                lowered by log N_ij, N_ij the number of rounds whose window
//                (and bucket, with SAME_BUCKET) gives key j to query i, so the
//                usual combination of the rounds is one softmax over the union.
//
// The work split and operand layouts follow k_attend_mfma: one workgroup of 4
// waves x 16 queries walks a range of chunks of one segment; the window's
// chunks sit in a ring of NS slots in LDS (NS = 3 with the look-ahead), qk rows
// row-major (keys, and the queries of the current chunk), v rows by pairs of
// 4-row groups (the A operand of P V); S^T = K Q^T per 16-key block, softmax
// in log2 units against the Cauchy-Schwarz bound, O^T = V^T P^T per 32-key
// step, row sums from a ones MFMA. Per key the slot also holds its bucket in
// this round and, for DEDUP, its chunk (and bucket) in every round, which the
// count N_ij compares with the query's. The next chunk's rows are loaded while
// the current one is computed. Per-round outputs are rows at original
// positions, fp16 (as the default kernel's) or fp32 with the fp32 flag; in the
// DOT form (the backward's recomputation) each query's row is reduced to
// dout(i) . o_r(i) instead, as in the default kernel's DOT form.
#include <type_traits>

#include "dedup_lanes.h"
#include "dtype.h"
#include "internal.h"
#include "rows_lds.h"
#include "walks.h"

namespace lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

using rows::BLay;
using rows::load_group;
using rows::store_pair;
using rows::store_rm;
using rows::zero_lds;

constexpr int kChunk = 64;
constexpr int kThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kBoundLimit = 60.0f;

template <int D, int NS, bool DD>
struct VLds {
  using L = BLay<D>;
  static constexpr int kKt = 0;                               // [NS][64] qk rows
  static constexpr int kVp = kKt + NS * L::kRM;               // [NS] v rows by group pairs
  static constexpr int kScale = kVp + NS * L::kPM;            // [NS][64] log2(e)/(sqrt(d)|k|)
  static constexpr int kPos = kScale + NS * kChunk * 4;       // [NS][64] original positions
  static constexpr int kBound = kPos + NS * kChunk * 4;       // [NS][64] log2(e)|k|/sqrt(d)
  static constexpr int kBkt = kBound + NS * kChunk * 4;       // [NS][64] bucket in the round
  // DEDUP: per key, its chunk (mod 2^16) and bucket in each of up to 8 rounds,
  // as 8 u16 lanes of 16 bytes
  static constexpr int kPack = DD ? 16 : 0;
  static constexpr int kCid = kBkt + NS * kChunk * 4;         // [NS][64] uint4
  static constexpr int kCbk = kCid + NS * kChunk * kPack;     // [NS][64] uint4
  static constexpr int kPn = kCbk + NS * kChunk * kPack;      // [64] next positions
  static constexpr int kBytes = kPn + kChunk * 4;
};

// one chunk's rows and per-row data between their loads and the staging
struct VRegs {
  uint4 k[4], v[4];
  int pos, bk;
  float n2;
  uint32_t cid[dedup::kMaxRounds / 2], cbk[dedup::kMaxRounds / 2];  // u16 lanes
};

__device__ __forceinline__ float sat16(float x) { return fminf(fmaxf(x, -65504.0f), 65504.0f); }

// With a window of two chunks, two workgroups fit a CU at d = 128 (76 KB of LDS
// with the de-duplication counts, 245 VGPRs): let each wave take half the
// register file.
// DOT: o receives per query the scalar dout(i) . o_r(i) ([seg, L] fp32;
// dout(i) . v_i for a query that saw only itself, whose output is v_i), dout
// being bf16 rows [B*H, L, D].
template <int D, bool CAUSAL, int NS, bool DD, typename OT, bool DOT>
__global__ __launch_bounds__(kThreads)
__attribute__((amdgpu_waves_per_eu(NS == 2 ? 2 : 1, NS == 2 ? 2 : 1))) void k_attend_var(
    const unsigned char* __restrict__ qk, const unsigned char* __restrict__ v,
    const int32_t* __restrict__ perm, const float* __restrict__ knorm,
    const uint16_t* __restrict__ bkt, const int32_t* __restrict__ inv, OT* __restrict__ o,
    float* __restrict__ lse, int L, int R, int nseg, int chunks_per_wg, int ranges,
    int group_segs, int64_t o_seg_rows, int flags, const unsigned char* __restrict__ dout) {
  static_assert(!DOT || std::is_same<OT, float>::value, "the DOT form writes fp32 scalars");
  using Lay = BLay<D>;
  using M = VLds<D, NS, DD>;
  constexpr int KS = D / 32, DT = D / 16;
  constexpr int NB = 4 * NS;  // 16-key blocks of the window
  constexpr int NE = 2 * NS;  // 32-key steps of P V
  extern __shared__ __align__(16) unsigned char lds[];
  const int nchunks = L / kChunk;
  int64_t seg;
  int range;
  walks::range_block(blockIdx.x, group_segs, ranges, nseg, seg, range);
  const int c0 = range * chunks_per_wg;
  const int c1 = min(nchunks, c0 + chunks_per_wg);
  if (c0 >= c1) return;
  // chunks the range stages: c0 - 1 .. c1 - 1 (+ c1 when looking ahead)
  const int fend = min(nchunks, c1 + NS - 2);
  const int64_t bh = seg / R;
  const int64_t row0 = bh * L;
  const int32_t* pm = perm + seg * L;
  const unsigned char* qkb = qk + row0 * D * 2;
  const unsigned char* vb = v + row0 * D * 2;
  const bool sb = (flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  const bool nq = (flags & LSH_ATTN_FLAG_NORM_QUERIES) != 0;
  constexpr bool dd = DD;
  float* kscale = (float*)(lds + M::kScale);
  int* kpos = (int*)(lds + M::kPos);
  float* kbound = (float*)(lds + M::kBound);
  int* kbk = (int*)(lds + M::kBkt);
  uint4* kcid = (uint4*)(lds + M::kCid);
  uint4* kcbk = (uint4*)(lds + M::kCbk);
  int* pn = (int*)(lds + M::kPn);
  const int t = threadIdx.x;
  const float sc = kLog2e / sqrtf((float)D);
  auto slot_of = [](int x) { return (x + NS) % NS; };

  auto fetch = [&](VRegs& r) {  // the chunk whose positions are in pn
    load_group<D>(r.k, qkb, pn);
    load_group<D>(r.v, vb, pn);
    if (t < kChunk) {
      r.pos = pn[t];
      r.n2 = knorm[row0 + r.pos];
      if (sb) r.bk = bkt[seg * L + r.pos];
      if (dd)
        dedup::row_lanes(inv + bh * R * L, bkt + bh * R * L, R, L, kChunk, r.pos, sb, r.cid,
                         r.cbk);
    }
  };
  auto stage = [&](const VRegs& r, int sl) {
    store_rm<D>(lds + M::kKt + sl * Lay::kRM, r.k);
    store_pair<D>(lds + M::kVp + sl * Lay::kPM, r.v);
    if (t < kChunk) {
      const float nrm = sqrtf(r.n2);
      kscale[sl * kChunk + t] = r.n2 > 0.f ? sc / nrm : 0.f;
      kpos[sl * kChunk + t] = r.pos;
      kbound[sl * kChunk + t] = sc * nrm;
      if (sb) kbk[sl * kChunk + t] = r.bk;
      if (dd) {
        kcid[sl * kChunk + t] = make_uint4(r.cid[0], r.cid[1], r.cid[2], r.cid[3]);
        kcbk[sl * kChunk + t] = make_uint4(r.cbk[0], r.cbk[1], r.cbk[2], r.cbk[3]);
      }
    }
  };

  // absent chunks (before the first, after the last) stay zero: finite
  // operands that every mask excludes
  zero_lds(lds, M::kPn);
  __syncthreads();
  VRegs r;
  for (int x = max(c0 - 1, 0); x < min(fend, c0 + NS - 1); ++x) {
    if (t < kChunk) pn[t] = pm[x * kChunk + t];
    __syncthreads();
    fetch(r);
    stage(r, slot_of(x));
    __syncthreads();
  }
  if (c0 + NS - 1 < fend && t < kChunk) pn[t] = pm[(c0 + NS - 1) * kChunk + t];
  __syncthreads();

  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
  const uint32_t ones_u[4] = {one2, one2, one2, one2};
  const bf16x8_t ones = *(const bf16x8_t*)ones_u;
  const bool la = NS == 3;
  int pnext = 0;

  for (int c = c0; c < c1; ++c) {
    const int f = c + NS - 1;  // the chunk loaded during this step
    const bool more = f < fend;
    if (more) {
      fetch(r);
      if (f + 1 < fend && t < kChunk) pnext = pm[(f + 1) * kChunk + t];
    }
    const int cur = slot_of(c);
    const int q = 16 * w + lq;
    const int posq = kpos[cur * kChunk + q];
    float mq = kbound[cur * kChunk + q];
    float rq = 1.0f;
    if (nq) {  // |q| = bound / sc; unit queries have bound sc
      rq = mq > 0.f ? sc / mq : 0.f;
      mq = mq > 0.f ? sc : 0.f;
    }
    const int bq = sb ? kbk[cur * kChunk + q] : 0;
    // the query's chunks and buckets over the rounds (lanes past R: 0)
    uint32_t qc[dedup::kMaxRounds / 2] = {0u, 0u, 0u, 0u}, qb[dedup::kMaxRounds / 2] = {0u, 0u, 0u, 0u};
    if (dd) {
      const uint4 c4 = kcid[cur * kChunk + q], b4 = kcbk[cur * kChunk + q];
      const uint32_t cw[4] = {c4.x, c4.y, c4.z, c4.w};
      dedup::query_lanes(cw, R, qc);
      qb[0] = b4.x, qb[1] = b4.y, qb[2] = b4.z, qb[3] = b4.w;
    }
    bf16x8_t qf[KS];
    {
      const unsigned char* row = lds + M::kKt + cur * Lay::kRM + q * Lay::kRow;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8_t*)(row + (32 * ks + 8 * g) * 2);
    }
    auto block_slot = [&](int kb) { return slot_of(c - 1 + kb / 4); };
    auto block_absent = [&](int kb) {
      const int x = c - 1 + kb / 4;
      return x < 0 || x >= nchunks;
    };
    auto qk_block = [&](int kb) -> floatx4_t {
      const unsigned char* row =
          lds + M::kKt + block_slot(kb) * Lay::kRM + ((kb & 3) * 16 + lq) * Lay::kRow;
      floatx4_t acc;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8_t*)(row + (32 * ks + 8 * g) * 2), qf[ks],
            ks == 0 ? floatx4_t{} : acc, 0, 0, 0);
      return acc;
    };
    // masks of the 4 keys 4g + 0..3 of block kb for this lane's query
    auto masks = [&](int kb, const int* kpv, bool* mk) {
      const int sl = block_slot(kb);
      const int key = (kb & 3) * 16 + 4 * g;
      const bool absent = block_absent(kb);
      int4 kb4 = {0, 0, 0, 0};
      if (sb) kb4 = *(const int4*)(kbk + sl * kChunk + key);
      const int kbv[4] = {kb4.x, kb4.y, kb4.z, kb4.w};
#pragma unroll
      for (int b = 0; b < 4; ++b)
        mk[b] = absent | (CAUSAL ? kpv[b] >= posq : kpv[b] == posq) | (sb && kbv[b] != bq);
    };
    // log2 N for key kk of slot sl: the rounds whose window (and bucket) give
    // it to this query
    auto log2_shared = [&](int sl, int kk) -> float {
      const uint4 c4 = kcid[sl * kChunk + kk];
      const uint32_t cw[4] = {c4.x, c4.y, c4.z, c4.w};
      uint4 b4 = {0u, 0u, 0u, 0u};
      if (sb) b4 = kcbk[sl * kChunk + kk];
      const uint32_t bw[4] = {b4.x, b4.y, b4.z, b4.w};
      return dedup::log2_rounds(qc, qb, cw, bw, R, la, sb);
    };
    if (__ballot(mq > kBoundLimit) != 0ull) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NB; ++kb) {
        const floatx4_t sv = qk_block(kb);
        const int sl = block_slot(kb);
        const int key = (kb & 3) * 16 + 4 * g;
        const float4 scv = *(const float4*)(kscale + sl * kChunk + key);
        const int4 kp = *(const int4*)(kpos + sl * kChunk + key);
        const float s4[4] = {scv.x, scv.y, scv.z, scv.w};
        const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
        bool mk[4];
        masks(kb, kpv, mk);
#pragma unroll
        for (int b = 0; b < 4; ++b) mx = fmaxf(mx, mk[b] ? -INFINITY : sv[b] * s4[b] * rq);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mq = mx == -INFINITY ? 0.f : mx;
    }
    float rowsum = 0.f;
    floatx4_t oacc[DT];
    floatx4_t lacc = floatx4_t{};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = floatx4_t{};
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      bf16x8_t pf;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kb = 2 * e + half;
        const floatx4_t sv = qk_block(kb);
        const int sl = block_slot(kb);
        const int key = (kb & 3) * 16 + 4 * g;
        const float4 scv = *(const float4*)(kscale + sl * kChunk + key);
        const int4 kp = *(const int4*)(kpos + sl * kChunk + key);
        const float s4[4] = {scv.x, scv.y, scv.z, scv.w};
        const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
        bool mk[4];
        masks(kb, kpv, mk);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          float x = fmaf(sv[b], s4[b] * rq, -mq);
          if (dd) x -= log2_shared(sl, key + b);
          const float pv = __builtin_amdgcn_exp2f(mk[b] ? -INFINITY : x);
          rowsum += pv;
          pf[4 * half + b] = (__bf16)pv;
        }
      }
      const int sl = slot_of(c - 1 + e / 2);
      // key pair g + 4 (e % 2) of the 32-key step's chunk
      const unsigned char* vp = lds + M::kVp + sl * Lay::kPM + (g + 4 * (e & 1)) * Lay::kPair +
                                (lq >> 3) * Lay::kBlk8 + (lq & 7) * 16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            *(const bf16x8_t*)(vp + dt * 2 * Lay::kBlk8), pf, oacc[dt], 0, 0, 0);
      lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lacc, 0, 0, 0);
    }
    rowsum += __shfl_xor(rowsum, 16);
    rowsum += __shfl_xor(rowsum, 32);
    {
      const float l = lacc[0];
      const bool seen = l > 0.f;
      const float invl = seen ? 1.0f / l : 0.f;
      OT* orow = o + (seg * o_seg_rows + posq) * D;
      if constexpr (DOT) {
        // lane group g holds dims 16 dt + 4g + 0..3 of the row, as dout's
        // 8-byte pieces; the four groups' partial sums are added across lanes
        const unsigned char* drow = dout + ((row0 + posq) * D + 4 * g) * 2;
        auto lo = [](uint32_t x) { return __uint_as_float(x << 16); };
        auto hi = [](uint32_t x) { return __uint_as_float(x & 0xFFFF0000u); };
        float dsum = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint2 z = *(const uint2*)(drow + 32 * dt);
          dsum = fmaf(oacc[dt][0], lo(z.x), dsum);
          dsum = fmaf(oacc[dt][1], hi(z.x), dsum);
          dsum = fmaf(oacc[dt][2], lo(z.y), dsum);
          dsum = fmaf(oacc[dt][3], hi(z.y), dsum);
        }
        dsum *= invl;
        if (!seen) {  // the round's output is v_i itself
          const unsigned char* vrow = vb + (posq * D + 4 * g) * 2;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint2 x = *(const uint2*)(vrow + 32 * dt);
            const uint2 z = *(const uint2*)(drow + 32 * dt);
            dsum = fmaf(lo(x.x), lo(z.x), dsum);
            dsum = fmaf(hi(x.x), hi(z.x), dsum);
            dsum = fmaf(lo(x.y), lo(z.y), dsum);
            dsum = fmaf(hi(x.y), hi(z.y), dsum);
          }
        }
        dsum += __shfl_xor(dsum, 16);
        dsum += __shfl_xor(dsum, 32);
        if (g == 0) o[seg * L + posq] = dsum;
      } else if constexpr (sizeof(OT) == 2) {
        // fp16: tiles t, t + 1 packed, odd and even 16-lane rows swapped, so
        // lane group g stores dims 16(t + g%2) + 8(g/2) + 0..7 (16 bytes)
        uint32_t pk[DT][2];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
          const f16x2_t lo = {(_Float16)sat16(oacc[dt][0] * invl), (_Float16)sat16(oacc[dt][1] * invl)};
          const f16x2_t hi = {(_Float16)sat16(oacc[dt][2] * invl), (_Float16)sat16(oacc[dt][3] * invl)};
          pk[dt][0] = __builtin_bit_cast(uint32_t, lo);
          pk[dt][1] = __builtin_bit_cast(uint32_t, hi);
        }
#pragma unroll
        for (int j = 0; j < DT / 2; ++j) {
          const auto r0 = __builtin_amdgcn_permlane16_swap(pk[2 * j][0], pk[2 * j + 1][0], false, false);
          const auto r1 = __builtin_amdgcn_permlane16_swap(pk[2 * j][1], pk[2 * j + 1][1], false, false);
          *(uint4*)(orow + 32 * j + 16 * (g & 1) + 8 * (g >> 1)) = make_uint4(r0[0], r1[0], r0[1], r1[1]);
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          *(float4*)(orow + 16 * dt + 4 * g) = make_float4(oacc[dt][0] * invl, oacc[dt][1] * invl,
                                                           oacc[dt][2] * invl, oacc[dt][3] * invl);
      }
      if (g == 0) lse[seg * L + posq] = seen ? (mq + __log2f(rowsum)) * kLn2 : kSelfLogit;
    }
    __syncthreads();  // every wave is done with the slot of chunk c - 1
    if (more) {
      stage(r, slot_of(f));
      if (f + 1 < fend && t < kChunk) pn[t] = pnext;
    }
    __syncthreads();
  }
}

constexpr int kRangeChunks = 16;
constexpr int kResidentBlocks = 256;

template <int D, bool CAUSAL, int NS, bool DD, typename OT, bool DOT>
void launch_one(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                const float* knorm, const uint16_t* bkt, const int32_t* inv, OT* o, float* lse,
                const void* dout, hipStream_t s) {
  constexpr int shmem = VLds<D, NS, DD>::kBytes;
  static bool configured[kMaxDevices] = {};
  if (first_on_device(configured)) {
    (void)hipFuncSetAttribute((const void*)k_attend_var<D, CAUSAL, NS, DD, OT, DOT>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
  }
  const int64_t nseg = p.nseg();
  const walks::RangeShape sh =
      walks::range_shape(p.L / kChunk, nseg, p.R, kRangeChunks, kResidentBlocks);
  hipLaunchKernelGGL((k_attend_var<D, CAUSAL, NS, DD, OT, DOT>), dim3((unsigned)sh.blocks),
                     dim3(kThreads), shmem, s, (const unsigned char*)qk,
                     (const unsigned char*)v, perm, knorm, bkt, inv, o, lse, p.L, p.R,
                     (int)nseg, sh.per, sh.ranges, sh.group_segs, p.o_seg_rows(),
                     p.flags & kVariantFlags, (const unsigned char*)dout);
}

template <int D, typename OT, bool DOT = false>
void launch_d(const Problem& p, const void* qk, const void* v, const int32_t* perm,
              const float* knorm, const uint16_t* bkt, const int32_t* inv, OT* o, float* lse,
              hipStream_t s, const void* dout = nullptr) {
  const bool ahead = (p.flags & LSH_ATTN_FLAG_LOOK_AHEAD) != 0;
  const bool dd = (p.flags & LSH_ATTN_FLAG_DEDUP) != 0;
  auto go = [&](auto causal, auto ns, auto ddv) {
    launch_one<D, decltype(causal)::value, decltype(ns)::value, decltype(ddv)::value, OT, DOT>(
        p, qk, v, perm, knorm, bkt, inv, o, lse, dout, s);
  };
  using T = std::true_type;
  using F = std::false_type;
  using N2 = std::integral_constant<int, 2>;
  using N3 = std::integral_constant<int, 3>;
  if (p.causal) {
    if (ahead) dd ? go(T{}, N3{}, T{}) : go(T{}, N3{}, F{});
    else dd ? go(T{}, N2{}, T{}) : go(T{}, N2{}, F{});
  } else {
    if (ahead) dd ? go(F{}, N3{}, T{}) : go(F{}, N3{}, F{});
    else dd ? go(F{}, N2{}, T{}) : go(F{}, N2{}, F{});
  }
}

}  // namespace

bool attend_variant_mfma_supported(const Problem& p) {
  // (the de-duplication compares chunks mod 2^16: at most 32768 chunks)
  return p.dtype == LSH_ATTN_BF16 && p.m == kChunk && (p.d == 64 || p.d == 128) &&
         (p.flags & kVariantFlags) &&
         (!(p.flags & LSH_ATTN_FLAG_DEDUP) || (p.R <= dedup::kMaxRounds && p.L / kChunk <= 32768));
}

hipError_t launch_attend_variant_mfma(const Problem& p, const void* qk, const void* v,
                                      const int32_t* perm, const float* knorm,
                                      const uint16_t* buckets, const int32_t* inv, void* o,
                                      float* lse, hipStream_t s) {
  if (round_outputs_half(p)) {
    if (p.d == 64) launch_d<64>(p, qk, v, perm, knorm, buckets, inv, (_Float16*)o, lse, s);
    else launch_d<128>(p, qk, v, perm, knorm, buckets, inv, (_Float16*)o, lse, s);
  } else {
    if (p.d == 64) launch_d<64>(p, qk, v, perm, knorm, buckets, inv, (float*)o, lse, s);
    else launch_d<128>(p, qk, v, perm, knorm, buckets, inv, (float*)o, lse, s);
  }
  return hipGetLastError();
}

hipError_t launch_attend_variant_dot(const Problem& p, const void* qk, const void* v,
                                     const int32_t* perm, const float* knorm, const void* dout,
                                     const uint16_t* buckets, const int32_t* inv, float* od,
                                     float* lse, hipStream_t s) {
  if (p.d == 64) launch_d<64, float, true>(p, qk, v, perm, knorm, buckets, inv, od, lse, s, dout);
  else launch_d<128, float, true>(p, qk, v, perm, knorm, buckets, inv, od, lse, s, dout);
  return hipGetLastError();
}

}  // namespace lsh
