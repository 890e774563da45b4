// attend_mfma.hip -- chunked look-one-back attention on gfx950 matrix cores.
//
// Same definition as the plain kernel in attend.hip (Reformer summary at
// p2.ttnews.xyz, LSH attention and shared-QK self-mask sections; overview at
// www.dtcms.com/a/488796.html, section 2.1: unit keys, 1/sqrt(d) scale, look
// at the neighbouring chunk, taken as the previous one), for bf16 inputs,
// chunk_len 64 and d in {64, 128}.
//
// One workgroup = 2 waves walks a range of consecutive chunks of one
// (batch, head, round) segment. Chunk rows are read from HBM through the
// permutation (the gather is fused into the load) and staged in LDS:
//   Kt : qk rows of the previous and current chunk, row-major (+16 B pad);
//        they are the keys and, for the current chunk, the queries (shared QK);
//   Vq : v rows stored as groups of 4 keys x d dims x 4 (8 bytes per dim), so
//        that one 8-byte LDS read yields 4 consecutive keys of one dim, the
//        B-operand layout of the P.V product;
//   per key: log2(e)/(sqrt(d) |k|), original position, and log2(e) |k|/sqrt(d).
// The previous chunk stays in LDS, so every chunk is loaded once per walk.
//
// Per wave (32 queries = 2 blocks of 16), v_mfma_f32_16x16x32_bf16:
//   S^T[key, query] = K Q^T over the 128-key window (64 for chunk 0);
//   lane l holds query l%16 of each block and keys 16kb + 4(l/16) + 0..3.
// Softmax in log2 units, p = exp2(s * scale_key - m_query). The shift m is the
// Cauchy-Schwarz bound |q| log2(e)/sqrt(d) >= every logit of the query (keys are
// unit vectors), so no max pass is needed; if a bound exceeds 60 (a query norm
// far outside the usual range) the wave takes the true row max instead, so
// exp2 never under- or overflows. Masked keys (causal: later original position;
// self) get p = 0. A query whose p are all 0 saw nothing but itself: its output
// is v_i and its logsumexp -1e5, as in the definition.
// P.V: the P block of the A operand comes straight from the S^T accumulators
// (their key order is the order of the A operand's k index), the B operand
// from Vq. An extra MFMA against a block of ones yields the row sums of the
// bf16-rounded P, so numerator and denominator use the same weights; the
// logsumexp takes the fp32 sum of the unrounded p.
#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;
constexpr int kThreads = 128;  // 2 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kBoundLimit = 60.0f;

template <int D>
struct Lds {
  static constexpr int kRow = D * 2 + 16;     // bytes per staged qk row
  static constexpr int kQuad = D * 8 + 32;    // bytes per group of 4 v rows
  static constexpr int kKt = 0;
  static constexpr int kVq = kKt + 2 * kChunk * kRow;
  static constexpr int kScale = kVq + 2 * (kChunk / 4) * kQuad;
  static constexpr int kPos = kScale + 2 * kChunk * 4;
  static constexpr int kBound = kPos + 2 * kChunk * 4;
  static constexpr int kBytes = kBound + 2 * kChunk * 4;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo).bits | ((uint32_t)f32_to_bf16(hi).bits << 16);
}

template <typename OT>
__device__ __forceinline__ void store_o(OT* p, float x);
template <>
__device__ __forceinline__ void store_o<float>(float* p, float x) { *p = x; }
template <>
__device__ __forceinline__ void store_o<_Float16>(_Float16* p, float x) {
  x = fminf(fmaxf(x, -65504.0f), 65504.0f);
  *p = (_Float16)x;
}

// Stage chunk `c` of segment `seg` into LDS slot `sl`.
template <int D>
__device__ __forceinline__ void load_chunk(unsigned char* lds, int sl, int c, const uint4* qk_rows,
                                           const uint4* v_rows, const int32_t* pm, int64_t row0,
                                           bool sorted, int64_t sorted_row0) {
  using Lay = Lds<D>;
  const int t = threadIdx.x;
  constexpr int kPieces = D * 2 / 16;  // uint4 per row
  // qk rows: thread t takes row t/2, half t%2
  {
    const int r = t >> 1, half = t & 1;
    const int pos = pm[c * kChunk + r];
    const uint4* src = sorted ? qk_rows + (sorted_row0 + c * kChunk + r) * kPieces
                              : qk_rows + (row0 + pos) * kPieces;
    uint4 x[kPieces / 2];
#pragma unroll
    for (int k = 0; k < kPieces / 2; ++k) x[k] = src[half * (kPieces / 2) + k];
    float nn = 0.f;
#pragma unroll
    for (int k = 0; k < kPieces / 2; ++k) {
      const uint32_t w[4] = {x[k].x, x[k].y, x[k].z, x[k].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float a = __uint_as_float(w[u] << 16), b = __uint_as_float(w[u] & 0xFFFF0000u);
        nn = fmaf(a, a, nn);
        nn = fmaf(b, b, nn);
      }
    }
    nn += __shfl_xor(nn, 1);
    uint4* dst = (uint4*)(lds + Lay::kKt + (sl * kChunk + r) * Lay::kRow) + half * (kPieces / 2);
#pragma unroll
    for (int k = 0; k < kPieces / 2; ++k) dst[k] = x[k];
    if (half == 0) {
      const float nrm = sqrtf(nn);
      const float sc = kLog2e / sqrtf((float)D);
      ((float*)(lds + Lay::kScale))[sl * kChunk + r] = nn > 0.f ? sc / nrm : 0.f;
      ((int*)(lds + Lay::kPos))[sl * kChunk + r] = pos;
      ((float*)(lds + Lay::kBound))[sl * kChunk + r] = sc * nrm;
    }
  }
  // v rows, 4 keys x 8 dims per piece, stored as [quad][dim][4 keys]
  {
    constexpr int kSegs = D / 8;                      // 8-dim pieces per row
    constexpr int kPer = kSegs * 16 / kThreads;       // pieces per thread (1 or 2)
#pragma unroll
    for (int pp = 0; pp < kPer; ++pp) {
      const int id = t + pp * kThreads;
      const int qd = id / kSegs, sg = id % kSegs;
      uint4 x[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int slot = c * kChunk + qd * 4 + k;
        const int64_t row = sorted ? sorted_row0 + slot : row0 + pm[slot];
        x[k] = v_rows[row * kPieces + sg];
      }
      uint2* dst = (uint2*)(lds + Lay::kVq + (sl * (kChunk / 4) + qd) * Lay::kQuad) + sg * 8;
      const uint32_t w0[4] = {x[0].x, x[0].y, x[0].z, x[0].w};
      const uint32_t w1[4] = {x[1].x, x[1].y, x[1].z, x[1].w};
      const uint32_t w2[4] = {x[2].x, x[2].y, x[2].z, x[2].w};
      const uint32_t w3[4] = {x[3].x, x[3].y, x[3].z, x[3].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        dst[2 * u] = make_uint2((w0[u] & 0xFFFFu) | (w1[u] << 16), (w2[u] & 0xFFFFu) | (w3[u] << 16));
        dst[2 * u + 1] = make_uint2((w0[u] >> 16) | (w1[u] & 0xFFFF0000u),
                                    (w2[u] >> 16) | (w3[u] & 0xFFFF0000u));
      }
    }
  }
}

template <int D, typename OT, bool CAUSAL>
__global__ __launch_bounds__(kThreads) void k_attend_mfma(
    const uint4* __restrict__ qk, const uint4* __restrict__ v, const uint4* __restrict__ qk_s,
    const uint4* __restrict__ v_s, const uint16_t* __restrict__ v_raw,
    const int32_t* __restrict__ perm, OT* __restrict__ o, float* __restrict__ lse, int L, int R,
    int nseg, int chunks_per_wg) {
  using Lay = Lds<D>;
  extern __shared__ __align__(16) unsigned char lds[];
  const int nchunks = L / kChunk;
  const int64_t seg = blockIdx.x % (unsigned)nseg;
  const int range = blockIdx.x / (unsigned)nseg;
  const int c0 = range * chunks_per_wg;
  const int c1 = min(nchunks, c0 + chunks_per_wg);
  if (c0 >= c1) return;
  const int64_t bh = seg / R;
  const int32_t* pm = perm + seg * L;
  const int64_t row0 = bh * L;           // first row of this (b, h) in qk / v
  const int64_t srow0 = seg * L;         // first row of this segment in the sorted copies
  const bool sorted = qk_s != nullptr;
  const uint4* qk_rows = sorted ? qk_s : qk;
  const uint4* v_rows = sorted ? v_s : v;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;     // lane group 0..3
  const int li = lane & 15;    // column within a 16-block

  if (c0 > 0) load_chunk<D>(lds, (c0 - 1) & 1, c0 - 1, qk_rows, v_rows, pm, row0, sorted, srow0);
  load_chunk<D>(lds, c0 & 1, c0, qk_rows, v_rows, pm, row0, sorted, srow0);
  __syncthreads();

  const float* kscale = (const float*)(lds + Lay::kScale);
  const int* kpos = (const int*)(lds + Lay::kPos);
  const float* kbound = (const float*)(lds + Lay::kBound);

  for (int c = c0; c < c1; ++c) {
    const int cur = c & 1, prv = cur ^ 1;
    const int kb0 = c > 0 ? 0 : 4;  // chunk 0 has no previous chunk
    // queries of this wave: 32w + 16qb + li
    bf16x8_t qf[2][D / 32];
    float mq[2];
    int posq[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      const int q = 32 * w + 16 * qb + li;
      const unsigned char* row = lds + Lay::kKt + (cur * kChunk + q) * Lay::kRow;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) qf[qb][ks] = *(const bf16x8_t*)(row + (ks * 32 + 8 * g) * 2);
      mq[qb] = kbound[cur * kChunk + q];
      posq[qb] = kpos[cur * kChunk + q];
    }
    // S^T = K Q^T
    floatx4_t s[8][2];
#pragma unroll
    for (int kb = 0; kb < 8; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 8; ++kb) {
      if (kb < kb0) continue;
      const int sl = kb < 4 ? prv : cur;
      const unsigned char* row = lds + Lay::kKt + (sl * kChunk + (kb & 3) * 16 + li) * Lay::kRow;
#pragma unroll
      for (int ks = 0; ks < D / 32; ++ks) {
        const bf16x8_t a = *(const bf16x8_t*)(row + (ks * 32 + 8 * g) * 2);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[qb][ks], s[kb][qb], 0, 0, 0);
      }
    }
    // softmax weights in log2 units
    const bool slow = __ballot(mq[0] > kBoundLimit || mq[1] > kBoundLimit) != 0ull;
    // key kb*16 + 4g + vv is masked for query block qb: absent (chunk 0 has no
    // previous chunk), the query itself, or (causal) a later original position
    auto masked = [&](int kb, int qb, int vv, int kp) -> bool {
      if (kb < kb0) return true;
      const bool self = (kb == 4 + 2 * w + qb) && (4 * g + vv == li);
      return self || (CAUSAL && kp > posq[qb]);
    };
    if (slow) {
      float mx[2] = {-INFINITY, -INFINITY};
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const int sl = kb < 4 ? prv : cur;
        const float4 sc = *(const float4*)(kscale + sl * kChunk + (kb & 3) * 16 + 4 * g);
        const int4 kp = *(const int4*)(kpos + sl * kChunk + (kb & 3) * 16 + 4 * g);
        const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
        const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int vv = 0; vv < 4; ++vv)
            if (!masked(kb, qb, vv, kpv[vv])) mx[qb] = fmaxf(mx[qb], s[kb][qb][vv] * scv[vv]);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        float m = fmaxf(mx[qb], __shfl_xor(mx[qb], 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        mq[qb] = m == -INFINITY ? 0.f : m;
      }
    }
    bf16x8_t pf[2][4];
    float rowsum[2] = {0.f, 0.f};  // fp32 sum of p, for the logsumexp
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      float p[2][8];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int kb = 2 * t + h;
        const int sl = kb < 4 ? prv : cur;
        const float4 sc = *(const float4*)(kscale + sl * kChunk + (kb & 3) * 16 + 4 * g);
        const int4 kp = *(const int4*)(kpos + sl * kChunk + (kb & 3) * 16 + 4 * g);
        const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
        const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int vv = 0; vv < 4; ++vv) {
            const float x = fmaf(s[kb][qb][vv], scv[vv], -mq[qb]);
            p[qb][4 * h + vv] = masked(kb, qb, vv, kpv[vv]) ? 0.f : __builtin_amdgcn_exp2f(x);
            rowsum[qb] += p[qb][4 * h + vv];
          }
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const uint32_t u[4] = {pack_bf16x2(p[qb][0], p[qb][1]), pack_bf16x2(p[qb][2], p[qb][3]),
                               pack_bf16x2(p[qb][4], p[qb][5]), pack_bf16x2(p[qb][6], p[qb][7])};
        pf[qb][t] = *(const bf16x8_t*)u;
      }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      rowsum[qb] += __shfl_xor(rowsum[qb], 16);
      rowsum[qb] += __shfl_xor(rowsum[qb], 32);
    }
    // O = P V, plus row sums against a block of ones
    floatx4_t acc[D / 16][2];
    floatx4_t lsum[2];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      lsum[qb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) acc[nt][qb] = floatx4_t{0.f, 0.f, 0.f, 0.f};
    }
    const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
    const uint32_t ones_u[4] = {one2, one2, one2, one2};
    const bf16x8_t ones = *(const bf16x8_t*)ones_u;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if (2 * t < kb0) continue;
      // keys 32t + 4g + 0..3 (quad 8t + g) and 32t + 16 + 4g + 0..3 (quad 8t + 4 + g)
      const int qa = 8 * t + g, qc = 8 * t + 4 + g;
      const unsigned char* va =
          lds + Lay::kVq + ((qa < 16 ? prv : cur) * (kChunk / 4) + (qa & 15)) * Lay::kQuad;
      const unsigned char* vc =
          lds + Lay::kVq + ((qc < 16 ? prv : cur) * (kChunk / 4) + (qc & 15)) * Lay::kQuad;
#pragma unroll
      for (int nt = 0; nt < D / 16; ++nt) {
        const int dim = nt * 16 + li;
        const uint2 lo = *(const uint2*)(va + dim * 8);
        const uint2 hi = *(const uint2*)(vc + dim * 8);
        const uint32_t u[4] = {lo.x, lo.y, hi.x, hi.y};
        const bf16x8_t b = *(const bf16x8_t*)u;
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          acc[nt][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[qb][t], b, acc[nt][qb], 0, 0, 0);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        lsum[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pf[qb][t], ones, lsum[qb], 0, 0, 0);
    }
    // normalise and scatter to original positions; lse per query
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
      for (int vv = 0; vv < 4; ++vv) {
        const int q = 32 * w + 16 * qb + 4 * g + vv;   // query row of this output element
        const int pos = kpos[cur * kChunk + q];
        const float l = lsum[qb][vv];
        const float m = __shfl(mq[qb], 4 * g + vv);
        const float lx = __shfl(rowsum[qb], 4 * g + vv);
        OT* orow = o + (seg * L + pos) * D;
        if (l > 0.f) {
          const float inv = 1.0f / l;
#pragma unroll
          for (int nt = 0; nt < D / 16; ++nt) store_o<OT>(orow + nt * 16 + li, acc[nt][qb][vv] * inv);
        } else {
          const uint16_t* vr = v_raw + (row0 + pos) * D;
#pragma unroll
          for (int nt = 0; nt < D / 16; ++nt)
            store_o<OT>(orow + nt * 16 + li, __uint_as_float((uint32_t)vr[nt * 16 + li] << 16));
        }
        if (li == vv) lse[seg * L + pos] = l > 0.f ? (m + __log2f(lx)) * kLn2 : kSelfLogit;
      }
    }
    __syncthreads();  // every wave is done with slot prv
    if (c + 1 < c1) {
      load_chunk<D>(lds, prv, c + 1, qk_rows, v_rows, pm, row0, sorted, srow0);
      __syncthreads();
    }
  }
}

template <int D, typename OT, bool CAUSAL>
void launch_one(const Problem& p, const void* qk, const void* v, const void* qk_s,
                const void* v_s, const int32_t* perm, OT* o, float* lse, hipStream_t s) {
  const int nchunks = p.L / kChunk;
  const int64_t nseg = p.nseg();
  const int64_t target = 1024;
  int64_t ranges = (target + nseg - 1) / nseg;
  if (ranges > nchunks) ranges = nchunks;
  if (ranges < 1) ranges = 1;
  const int per = (int)((nchunks + ranges - 1) / ranges);
  ranges = (nchunks + per - 1) / per;
  const size_t shmem = Lds<D>::kBytes;
  hipLaunchKernelGGL((k_attend_mfma<D, OT, CAUSAL>), dim3((unsigned)(nseg * ranges)),
                     dim3(kThreads), shmem, s, (const uint4*)qk, (const uint4*)v,
                     (const uint4*)qk_s, (const uint4*)v_s, (const uint16_t*)v, perm, o, lse, p.L,
                     p.R, (int)nseg, per);
}

template <int D, typename OT>
void launch_d(const Problem& p, const void* qk, const void* v, const void* qk_s, const void* v_s,
              const int32_t* perm, OT* o, float* lse, hipStream_t s) {
  if (p.causal) launch_one<D, OT, true>(p, qk, v, qk_s, v_s, perm, o, lse, s);
  else launch_one<D, OT, false>(p, qk, v, qk_s, v_s, perm, o, lse, s);
}

}  // namespace

bool attend_mfma_supported(const Problem& p) {
  return p.dtype == LSH_ATTN_BF16 && p.m == kChunk && (p.d == 64 || p.d == 128);
}

template <typename OT>
hipError_t launch_attend_mfma(const Problem& p, const void* qk, const void* v,
                              const void* qk_sorted, const void* v_sorted, const int32_t* perm,
                              OT* o, float* lse, hipStream_t s) {
  static bool configured = false;
  if (!configured) {
    // allow the dynamic LDS size above the 64 KiB default
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, true>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, false>,
                        hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    configured = true;
  }
  if (p.d == 64) launch_d<64, OT>(p, qk, v, qk_sorted, v_sorted, perm, o, lse, s);
  else launch_d<128, OT>(p, qk, v, qk_sorted, v_sorted, perm, o, lse, s);
  return hipGetLastError();
}

template hipError_t launch_attend_mfma<float>(const Problem&, const void*, const void*, const void*,
                                              const void*, const int32_t*, float*, float*,
                                              hipStream_t);
template hipError_t launch_attend_mfma<_Float16>(const Problem&, const void*, const void*,
                                                 const void*, const void*, const int32_t*,
                                                 _Float16*, float*, hipStream_t);

}  // namespace lsh
