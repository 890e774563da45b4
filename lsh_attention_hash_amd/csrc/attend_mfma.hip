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
//        that one 8-byte LDS read yields 4 consecutive keys of one dim;
//   per key: log2(e)/(sqrt(d) |k|), original position, and log2(e) |k|/sqrt(d).
// The previous chunk stays in LDS, so every chunk is loaded once per walk.
// The rows of chunk c+1 are loaded while chunk c is computed, addressed by
// its positions that the previous step staged in LDS; the positions of chunk
// c+2 are loaded at the same time. Both are waited for only when chunk c+1
// is staged, after the compute, so no wait at the top of a step involves
// memory (loads and stores share one completion counter).
//
// Per wave (32 queries), v_mfma_f32_32x32x16_bf16:
//   S^T[key, query] = K Q^T over the 128-key window (64 for chunk 0), 4
//   blocks of 32 keys; lane l holds query l%32 and keys
//   32kb + 8(v/4) + 4(l/32) + v%4, v = 0..15, of every block.
// Softmax in log2 units, p = exp2(s * scale_key - m_query), masked keys
// entering exp2 as -inf (no branches). The shift m is the
// Cauchy-Schwarz bound |q| log2(e)/sqrt(d) >= every logit of the query (keys are
// unit vectors), so no max pass is needed; if a bound exceeds 60 (a query norm
// far outside the usual range) the wave takes the true row max instead, so
// exp2 never under- or overflows. Masked keys (causal: later original position;
// self) get p = 0. A query whose p are all 0 saw nothing but itself: its
// logsumexp is -1e5, as in the definition, and its output for the round (v_i)
// is not written here; the round combination reads v_i for such rounds.
// O^T = V^T P^T: the B operand (P^T) comes straight from the S^T accumulators,
// with the k index of each 16-key step ordered as the accumulator registers
// (v = 8e..8e+7 of block kb), and the A operand (V^T) from two 8-byte Vq reads
// in the same key order. In the output, lane l holds 4 consecutive dims of
// query l%32 per register group, so each store writes 8 (fp16) or 16 (fp32)
// contiguous bytes. An MFMA against a block of ones gives the row sums of the
// bf16-rounded P, so numerator and denominator use the same weights; the
// logsumexp takes the fp32 sum of the unrounded p.
#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx16_t __attribute__((ext_vector_type(16)));

constexpr int kChunk = 64;
constexpr int kThreads = 128;  // 2 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kBoundLimit = 60.0f;

template <int D>
struct Lds {
  static constexpr int kRow = D * 2 + 16;     // bytes per staged qk row
  static constexpr int kQuad = D * 8 + 128;   // bytes per group of 4 v rows (+128: the two
                                              // lane halves of a read hit disjoint banks)
  static constexpr int kKt = 0;
  static constexpr int kVq = kKt + 2 * kChunk * kRow;
  static constexpr int kScale = kVq + 2 * (kChunk / 4) * kQuad;
  static constexpr int kPos = kScale + 2 * kChunk * 4;
  static constexpr int kBound = kPos + 2 * kChunk * 4;
  static constexpr int kPermNext = kBound + 2 * kChunk * 4;  // positions of the next chunk
  static constexpr int kBytes = kPermNext + kChunk * 4;
};

// 4 consecutive outputs packed into 32-bit words (fp16: 2 words, fp32: 4)
template <typename OT>
struct Pack4 {
  static constexpr int kWords = 4 * (int)sizeof(OT) / 4;
};
__device__ __forceinline__ float sat16(float x) { return fminf(fmaxf(x, -65504.0f), 65504.0f); }
__device__ __forceinline__ void pack4(float a, float b, float c, float d, uint32_t* w, float*) {
  w[0] = __float_as_uint(a); w[1] = __float_as_uint(b);
  w[2] = __float_as_uint(c); w[3] = __float_as_uint(d);
}
__device__ __forceinline__ void pack4(float a, float b, float c, float d, uint32_t* w, _Float16*) {
  typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
  const f16x2_t lo = {(_Float16)sat16(a), (_Float16)sat16(b)};
  const f16x2_t hi = {(_Float16)sat16(c), (_Float16)sat16(d)};
  w[0] = __builtin_bit_cast(uint32_t, lo);
  w[1] = __builtin_bit_cast(uint32_t, hi);
}
// 8 consecutive outputs from two packed groups of 4
template <typename OT>
__device__ __forceinline__ void store8(OT* p, const uint32_t* lo, const uint32_t* hi) {
  constexpr int W = Pack4<OT>::kWords;
  uint32_t u[2 * W];
#pragma unroll
  for (int i = 0; i < W; ++i) {
    u[i] = lo[i];
    u[W + i] = hi[i];
  }
#pragma unroll
  for (int i = 0; i < 2 * W; i += 4) *(uint4*)((uint32_t*)p + i) = make_uint4(u[i], u[i + 1], u[i + 2], u[i + 3]);
}

// Thread t loads half t%2 of qk row t/2 and, for piece pp, 8 dims of the 4 v
// rows of group (t + 128 pp) / (D/8).
template <int D>
struct ChunkRegs {
  static constexpr int kPieces = D * 2 / 16;  // uint4 per row
  static constexpr int kSegs = D / 8;         // 8-dim pieces per row
  static constexpr int kPer = kSegs * 16 / kThreads;
  uint4 qk[kPieces / 2];
  uint4 v[kPer][4];
  int pos;
  float n2;  // squared norm of qk row t/2
};

// permutation entries (original positions) a chunk's loads need
template <int D>
struct PermRegs {
  int pos;
  int vpos[ChunkRegs<D>::kPer][4];
};

// The entries come from the chunk's 64 positions staged in LDS.
template <int D>
__device__ __forceinline__ void read_perm(PermRegs<D>& pr, const int* pn) {
  using CR = ChunkRegs<D>;
  const int t = threadIdx.x;
  pr.pos = pn[t >> 1];
#pragma unroll
  for (int pp = 0; pp < CR::kPer; ++pp) {
    const int qd = (t + pp * kThreads) / CR::kSegs;
    const int4 q4 = *(const int4*)(pn + qd * 4);
    pr.vpos[pp][0] = q4.x;
    pr.vpos[pp][1] = q4.y;
    pr.vpos[pp][2] = q4.z;
    pr.vpos[pp][3] = q4.w;
  }
}

// Rows are addressed as a wave-uniform base (the segment's first row) plus a
// 32-bit byte offset per lane, every offset computed before the first load,
// so no load waits for an earlier one to release its address registers.
template <int D, bool SORTED>
__device__ __forceinline__ void fetch_rows(ChunkRegs<D>& cr, const PermRegs<D>& pr, int c,
                                           const uint4* qk_rows, const uint4* v_rows,
                                           const float* knorm, int64_t row0,
                                           int64_t sorted_row0) {
  constexpr bool sorted = SORTED;
  using CR = ChunkRegs<D>;
  constexpr uint32_t kRowBytes = D * 2;
  const int t = threadIdx.x;
  const int64_t base_row = sorted ? sorted_row0 + c * kChunk : row0;
  const unsigned char* qb = (const unsigned char*)(qk_rows + base_row * CR::kPieces);
  const unsigned char* vb = (const unsigned char*)(v_rows + base_row * CR::kPieces);
  const int r = t >> 1, half = t & 1;
  const uint32_t qoff = (uint32_t)(sorted ? r : pr.pos) * kRowBytes + half * (kRowBytes / 2);
  uint32_t voff[CR::kPer][4];
#pragma unroll
  for (int pp = 0; pp < CR::kPer; ++pp) {
    const int id = t + pp * kThreads;
    const int qd = id / CR::kSegs, sg = id % CR::kSegs;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      voff[pp][k] = (uint32_t)(sorted ? qd * 4 + k : pr.vpos[pp][k]) * kRowBytes + sg * 16;
  }
  cr.pos = pr.pos;
  __builtin_amdgcn_sched_barrier(0);
  cr.n2 = knorm[row0 + pr.pos];
#pragma unroll
  for (int k = 0; k < CR::kPieces / 2; ++k) cr.qk[k] = *(const uint4*)(qb + qoff + k * 16);
#pragma unroll
  for (int pp = 0; pp < CR::kPer; ++pp)
#pragma unroll
    for (int k = 0; k < 4; ++k) cr.v[pp][k] = *(const uint4*)(vb + voff[pp][k]);
}

template <int D>
__device__ __forceinline__ void stage_chunk(unsigned char* lds, int sl, const ChunkRegs<D>& cr) {
  using Lay = Lds<D>;
  using CR = ChunkRegs<D>;
  const int t = threadIdx.x;
  {
    const int r = t >> 1, half = t & 1;
    const float nn = cr.n2;
    uint4* dst = (uint4*)(lds + Lay::kKt + (sl * kChunk + r) * Lay::kRow) + half * (CR::kPieces / 2);
    // (each piece passes through a register-only asm statement, so the copy
    // cannot become a memcpy from a stack copy of the registers)
#pragma unroll
    for (int k = 0; k < CR::kPieces / 2; ++k) {
      uint4 x = cr.qk[k];
      asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
      dst[k] = x;
    }
    if (half == 0) {
      const float nrm = sqrtf(nn);
      const float sc = kLog2e / sqrtf((float)D);
      ((float*)(lds + Lay::kScale))[sl * kChunk + r] = nn > 0.f ? sc / nrm : 0.f;
      ((int*)(lds + Lay::kPos))[sl * kChunk + r] = cr.pos;
      ((float*)(lds + Lay::kBound))[sl * kChunk + r] = sc * nrm;
    }
  }
  // v rows, 4 keys x 8 dims per piece, stored as [quad][dim][4 keys]
#pragma unroll
  for (int pp = 0; pp < CR::kPer; ++pp) {
    const int id = t + pp * kThreads;
    const int qd = id / CR::kSegs, sg = id % CR::kSegs;
    uint2* dst = (uint2*)(lds + Lay::kVq + (sl * (kChunk / 4) + qd) * Lay::kQuad) + sg * 8;
    const uint32_t w0[4] = {cr.v[pp][0].x, cr.v[pp][0].y, cr.v[pp][0].z, cr.v[pp][0].w};
    const uint32_t w1[4] = {cr.v[pp][1].x, cr.v[pp][1].y, cr.v[pp][1].z, cr.v[pp][1].w};
    const uint32_t w2[4] = {cr.v[pp][2].x, cr.v[pp][2].y, cr.v[pp][2].z, cr.v[pp][2].w};
    const uint32_t w3[4] = {cr.v[pp][3].x, cr.v[pp][3].y, cr.v[pp][3].z, cr.v[pp][3].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      dst[2 * u] = make_uint2((w0[u] & 0xFFFFu) | (w1[u] << 16), (w2[u] & 0xFFFFu) | (w3[u] << 16));
      dst[2 * u + 1] = make_uint2((w0[u] >> 16) | (w1[u] & 0xFFFF0000u),
                                  (w2[u] >> 16) | (w3[u] & 0xFFFF0000u));
    }
  }
}

// LDS (the two chunks of K and V) allows one wave per SIMD at d = 128, so the
// register budget is the whole file; say so, or the compiler aims for two
// waves and spills.
template <int D, typename OT, bool CAUSAL, bool SORTED>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void k_attend_mfma(
    const uint4* __restrict__ qk, const uint4* __restrict__ v, const uint4* __restrict__ qk_s,
    const uint4* __restrict__ v_s, const int32_t* __restrict__ perm,
    const float* __restrict__ knorm, OT* __restrict__ o, float* __restrict__ lse, int L, int R,
    int nseg, int chunks_per_wg) {
  using Lay = Lds<D>;
  constexpr int KS = D / 16;       // 16-dim K-steps of QK^T
  constexpr int MB = D / 32;       // 32-dim blocks of the output
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
  const uint4* qk_rows = SORTED ? qk_s : qk;
  const uint4* v_rows = SORTED ? v_s : v;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int h = lane >> 5;     // lane half
  const int lq = lane & 31;    // query (column) of this lane within the wave's 32

  ChunkRegs<D> cr;
  PermRegs<D> pr;
  int* pn = (int*)(lds + Lay::kPermNext);
  // positions of chunk c into LDS (threads 0..63), for the prologue
  auto perm_to_lds = [&](int c) {
    if (threadIdx.x < kChunk) pn[threadIdx.x] = pm[c * kChunk + threadIdx.x];
  };
  if (c0 > 0) {
    perm_to_lds(c0 - 1);
    __syncthreads();
    read_perm<D>(pr, pn);
    fetch_rows<D, SORTED>(cr, pr, c0 - 1, qk_rows, v_rows, knorm, row0, srow0);
    stage_chunk<D>(lds, (c0 - 1) & 1, cr);
    __syncthreads();
  } else {
    // Chunk 0 has no previous chunk: its slot holds zero keys and values, so
    // the window's first 64 logits are finite (0) and contribute nothing once
    // masked as absent; the loops then need no branch for chunk 0.
    uint4* kt = (uint4*)(lds + Lay::kKt + kChunk * Lay::kRow);        // slot 1
    for (int i = threadIdx.x; i < kChunk * Lay::kRow / 16; i += kThreads) kt[i] = uint4{};
    uint4* vq = (uint4*)(lds + Lay::kVq + (kChunk / 4) * Lay::kQuad);  // slot 1
    for (int i = threadIdx.x; i < (kChunk / 4) * Lay::kQuad / 16; i += kThreads) vq[i] = uint4{};
    if (threadIdx.x < kChunk) ((float*)(lds + Lay::kScale))[kChunk + threadIdx.x] = 0.f;
  }
  perm_to_lds(c0);
  __syncthreads();
  read_perm<D>(pr, pn);
  fetch_rows<D, SORTED>(cr, pr, c0, qk_rows, v_rows, knorm, row0, srow0);
  stage_chunk<D>(lds, c0 & 1, cr);
  __syncthreads();
  if (c0 + 1 < c1) perm_to_lds(c0 + 1);
  __syncthreads();
  int pnext = 0;  // a position of chunk c + 2, in flight to LDS

  const float* kscale = (const float*)(lds + Lay::kScale);
  const int* kpos = (const int*)(lds + Lay::kPos);
  const float* kbound = (const float*)(lds + Lay::kBound);
  const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
  const uint32_t ones_u[4] = {one2, one2, one2, one2};
  const bf16x8_t ones = *(const bf16x8_t*)ones_u;

  constexpr int W = Pack4<OT>::kWords;

  for (int c = c0; c < c1; ++c) {
    // Rows of chunk c + 1 (positions from LDS) and the positions of chunk
    // c + 2 are loaded while this chunk is computed; they are waited for only
    // when chunk c + 1 is staged, after the compute.
    if (c + 1 < c1) {
      read_perm<D>(pr, pn);
      fetch_rows<D, SORTED>(cr, pr, c + 1, qk_rows, v_rows, knorm, row0, srow0);
      if (c + 2 < c1 && threadIdx.x < kChunk) pnext = pm[(c + 2) * kChunk + threadIdx.x];
    }
    const int cur = c & 1, prv = cur ^ 1;
    const int kb0 = c > 0 ? 0 : 2;  // chunk 0 has no previous chunk
    const int q = 32 * w + lq;      // this lane's query row in the chunk
    float mq = kbound[cur * kChunk + q];
    const int posq = kpos[cur * kChunk + q];
    // S^T = K Q^T; K index of each step: dims h*D/2 + 8ks + 0..7 in both operands
    bf16x8_t qf[KS];
    {
      const unsigned char* row = lds + Lay::kKt + (cur * kChunk + q) * Lay::kRow + h * D;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8_t*)(row + ks * 16);
    }
    // S^T of key block kb (32 keys: window keys 32kb .. 32kb + 31)
    auto qk_block = [&](int kb) -> floatx16_t {
      const int sl = kb < 2 ? prv : cur;
      const unsigned char* row =
          lds + Lay::kKt + (sl * kChunk + (kb & 1) * 32 + lq) * Lay::kRow + h * D;
      floatx16_t acc;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *(const bf16x8_t*)(row + ks * 16);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[ks], ks == 0 ? floatx16_t{} : acc,
                                                       0, 0, 0);
      }
      return acc;
    };
    // A key is masked when it is absent (chunk 0 has no previous chunk), the
    // query itself, or (causal) at a later original position. Positions are
    // unique within a segment, so "itself" is pos_j == pos_q and the causal
    // and self masks together are pos_j >= pos_q.
    auto masked = [&](bool absent, int kp) -> bool {
      return absent || (CAUSAL ? kp >= posq : kp == posq);
    };
    // If a bound is far above the logits it bounds, shift by the true row
    // max instead (an extra QK^T pass; the bound depends only on the query,
    // so the choice is known before any product).
    if (__ballot(mq > kBoundLimit) != 0ull) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const floatx16_t sb = qk_block(kb);
        const int sl = kb < 2 ? prv : cur;
        const bool absent = kb < kb0;
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int key = (kb & 1) * 32 + 8 * a4 + 4 * h;
          const float4 sc = *(const float4*)(kscale + sl * kChunk + key);
          const int4 kp = *(const int4*)(kpos + sl * kChunk + key);
          const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
          const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
          for (int b = 0; b < 4; ++b) {
            const float x = sb[4 * a4 + b] * scv[b];
            mx = fmaxf(mx, masked(absent, kpv[b]) ? -INFINITY : x);
          }
        }
      }
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mq = mx == -INFINITY ? 0.f : mx;
    }
    // p of key block kb in bf16 as the B operand of O^T: step e takes the
    // accumulator registers v = 8e..8e+7
    float rowsum = 0.f;
    auto soft_block = [&](int kb, const floatx16_t& sb, bf16x8_t* pf) {
      const int sl = kb < 2 ? prv : cur;
      const bool absent = kb < kb0;
      float pv[16];
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int key = (kb & 1) * 32 + 8 * a4 + 4 * h;
        const float4 sc = *(const float4*)(kscale + sl * kChunk + key);
        const int4 kp = *(const int4*)(kpos + sl * kChunk + key);
        const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
        const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int vv = 4 * a4 + b;
          const float x = fmaf(sb[vv], scv[b], -mq);
          pv[vv] = __builtin_amdgcn_exp2f(masked(absent, kpv[b]) ? -INFINITY : x);
          rowsum += pv[vv];
        }
      }
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        bf16x8_t t;
#pragma unroll
        for (int j = 0; j < 8; ++j) t[j] = (__bf16)pv[8 * e + j];
        pf[e] = t;
      }
    };
    // O^T += V^T P^T over key block kb (+ row sums against ones)
    floatx16_t oacc[MB];
    floatx16_t lacc = floatx16_t{};
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) oacc[mb] = floatx16_t{};
    auto pv_block = [&](int kb, const bf16x8_t* pf) {
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        // keys 32kb + 16e + 4h + 0..3 and 32kb + 16e + 8 + 4h + 0..3 (window order)
        const int qa = 8 * kb + 4 * e + h, qc = qa + 2;
        const unsigned char* va =
            lds + Lay::kVq + ((qa < 16 ? prv : cur) * (kChunk / 4) + (qa & 15)) * Lay::kQuad;
        const unsigned char* vc =
            lds + Lay::kVq + ((qc < 16 ? prv : cur) * (kChunk / 4) + (qc & 15)) * Lay::kQuad;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) {
          const int dim = mb * 32 + lq;
          const uint2 lo = *(const uint2*)(va + dim * 8);
          const uint2 hi = *(const uint2*)(vc + dim * 8);
          const uint32_t u[4] = {lo.x, lo.y, hi.x, hi.y};
          oacc[mb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8_t*)u, pf[e],
                                                              oacc[mb], 0, 0, 0);
        }
        lacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ones, pf[e], lacc, 0, 0, 0);
      }
    };
    // Software pipeline over the four key blocks: the QK^T MFMAs of block
    // kb + 1 and the PV MFMAs of block kb - 1 run while the vector unit does
    // the softmax of block kb.
    {
      bf16x8_t pfa[2], pfb[2];
      floatx16_t s0 = qk_block(0);
      floatx16_t s1 = qk_block(1);
      soft_block(0, s0, pfa);
      floatx16_t s2 = qk_block(2);
      soft_block(1, s1, pfb);
      pv_block(0, pfa);

      floatx16_t s3 = qk_block(3);
      soft_block(2, s2, pfa);
      pv_block(1, pfb);
      soft_block(3, s3, pfb);
      pv_block(2, pfa);
      pv_block(3, pfb);
    }
    rowsum += __shfl_xor(rowsum, 32);
    // The next chunk, whose rows were loaded during this compute, is staged
    // before this chunk's outputs are stored: a wait on those loads then does
    // not also wait on the stores (one counter tracks both).
    __syncthreads();  // every wave is done with slot prv
    if (c + 1 < c1) {
      stage_chunk<D>(lds, prv, cr);
      if (c + 2 < c1 && threadIdx.x < kChunk) pn[threadIdx.x] = pnext;
    }
    // Normalise and scatter to the query's original position. Lane half h
    // holds dims 8a + 4h + 0..3 (a = 0..3) of each 32-dim block; one swap of
    // the lanes' upper and lower halves gives lane half h dims 16j + 8h + 0..7
    // (j = 0, 1), so each store writes 8 contiguous outputs. Every packed
    // output sits in its own register before the first store.
    const float l = lacc[0];
    const bool seen = l > 0.f;  // both lanes of a query agree
    uint32_t lo[MB][2][W], hi[MB][2][W];
    {
      const float inv = seen ? 1.0f / l : 0.f;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        uint32_t wa[4][W];
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4)
          pack4(oacc[mb][4 * a4] * inv, oacc[mb][4 * a4 + 1] * inv, oacc[mb][4 * a4 + 2] * inv,
                oacc[mb][4 * a4 + 3] * inv, wa[a4], (OT*)nullptr);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          // upper lanes send group 2j, lower lanes send group 2j + 1
#pragma unroll
          for (int i = 0; i < W; ++i) {
            const auto r = __builtin_amdgcn_permlane32_swap(wa[2 * j][i], wa[2 * j + 1][i],
                                                            false, false);
            lo[mb][j][i] = h ? r[0] : wa[2 * j][i];
            hi[mb][j][i] = h ? wa[2 * j + 1][i] : r[1];
          }
        }
      }
    }
    // A query that saw only itself (l == 0) has no row here: its output for
    // this round is v_i, which the round combination takes from v directly
    // (the logsumexp -1e5 marks the round).
    {
      OT* orow = o + (seg * L + posq) * D;
      if (seen) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int j = 0; j < 2; ++j) store8(orow + mb * 32 + 16 * j + 8 * h, lo[mb][j], hi[mb][j]);
      }
      if (h == 0) lse[seg * L + posq] = seen ? (mq + __log2f(rowsum)) * kLn2 : kSelfLogit;
    }
    __syncthreads();
  }
}

template <int D, typename OT, bool CAUSAL, bool SORTED>
void launch_one(const Problem& p, const void* qk, const void* v, const void* qk_s,
                const void* v_s, const int32_t* perm, const float* knorm, OT* o, float* lse, hipStream_t s) {
  const int nchunks = p.L / kChunk;
  const int64_t nseg = p.nseg();
  const int64_t target = 1024;
  int64_t ranges = (target + nseg - 1) / nseg;
  if (ranges > nchunks) ranges = nchunks;
  if (ranges < 1) ranges = 1;
  const int per = (int)((nchunks + ranges - 1) / ranges);
  ranges = (nchunks + per - 1) / per;
  const size_t shmem = Lds<D>::kBytes;
  hipLaunchKernelGGL((k_attend_mfma<D, OT, CAUSAL, SORTED>), dim3((unsigned)(nseg * ranges)),
                     dim3(kThreads), shmem, s, (const uint4*)qk, (const uint4*)v,
                     (const uint4*)qk_s, (const uint4*)v_s, perm, knorm, o, lse, p.L,
                     p.R, (int)nseg, per);
}

template <int D, typename OT>
void launch_d(const Problem& p, const void* qk, const void* v, const void* qk_s, const void* v_s,
              const int32_t* perm, const float* knorm, OT* o, float* lse, hipStream_t s) {
  const bool sorted = qk_s != nullptr;
  if (p.causal) {
    if (sorted) launch_one<D, OT, true, true>(p, qk, v, qk_s, v_s, perm, knorm, o, lse, s);
    else launch_one<D, OT, true, false>(p, qk, v, qk_s, v_s, perm, knorm, o, lse, s);
  } else {
    if (sorted) launch_one<D, OT, false, true>(p, qk, v, qk_s, v_s, perm, knorm, o, lse, s);
    else launch_one<D, OT, false, false>(p, qk, v, qk_s, v_s, perm, knorm, o, lse, s);
  }
}

}  // namespace

bool attend_mfma_supported(const Problem& p) {
  return p.dtype == LSH_ATTN_BF16 && p.m == kChunk && (p.d == 64 || p.d == 128);
}

template <typename OT>
hipError_t launch_attend_mfma(const Problem& p, const void* qk, const void* v,
                              const void* qk_sorted, const void* v_sorted, const int32_t* perm,
                              const float* knorm, OT* o, float* lse, hipStream_t s) {
  static bool configured = false;
  if (!configured) {
    // allow the dynamic LDS size above the 64 KiB default
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, true, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, false, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, true, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, false, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    configured = true;
  }
  if (p.d == 64) launch_d<64, OT>(p, qk, v, qk_sorted, v_sorted, perm, knorm, o, lse, s);
  else launch_d<128, OT>(p, qk, v, qk_sorted, v_sorted, perm, knorm, o, lse, s);
  return hipGetLastError();
}

template hipError_t launch_attend_mfma<float>(const Problem&, const void*, const void*, const void*,
                                              const void*, const int32_t*, const float*, float*,
                                              float*, hipStream_t);
template hipError_t launch_attend_mfma<_Float16>(const Problem&, const void*, const void*,
                                                 const void*, const void*, const int32_t*,
                                                 const float*, _Float16*, float*, hipStream_t);

}  // namespace lsh
