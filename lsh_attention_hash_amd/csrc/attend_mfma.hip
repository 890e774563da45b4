// attend_mfma.hip -- chunked look-one-back attention on gfx950 matrix cores.
//
// Same definition as the plain kernel in attend.hip (Reformer summary at
// p2.ttnews.xyz, LSH attention and shared-QK self-mask sections; overview at
// www.dtcms.com/a/488796.html, section 2.1: unit keys, 1/sqrt(d) scale, look
// at the neighbouring chunk, taken as the previous one), for bf16 inputs,
// chunk_len 64 and d in {64, 128}.
//
// One workgroup = 4 waves walks a range of consecutive chunks of one
// (batch, head, round) segment. Chunk rows are read from HBM through the
// permutation (the gather is fused into the load) and staged in LDS:
//   Kt : qk rows of the previous and current chunk, row-major (+16 B pad);
//        they are the keys and, for the current chunk, the queries (shared QK);
//   Vp : v rows stored by key pairs of 4-key groups (a, a + 4), a in
//        {0..3, 8..11}: per dim 16 bytes, the 4 keys of group a then those of
//        group a + 4, so one 16-byte LDS read is a whole A operand of PV (a
//        16-byte pad after every 8 dims keeps the staging writes and the
//        reads free of bank conflicts);
//   per key: log2(e)/(sqrt(d) |k|), original position, and log2(e) |k|/sqrt(d).
// The previous chunk stays in LDS, so every chunk is loaded once per walk.
// The rows of chunk c+1 are loaded while chunk c is computed, addressed by
// its positions that the previous step staged in LDS; the positions of chunk
// c+2 are loaded at the same time. Both are waited for only when chunk c+1
// is staged, after the compute, so no wait at the top of a step involves
// memory (loads and stores share one completion counter). The LDS of one
// workgroup (73 KB at d = 128) lets two share a CU, so each SIMD runs two
// waves, one of which computes while the other waits.
//
// Per wave (16 queries), v_mfma_f32_16x16x32_bf16:
//   S^T[key, query] = K Q^T over the 128-key window (64 for chunk 0), 8
//   blocks of 16 keys; lane l holds query l%16 and keys 4(l/16) + v,
//   v = 0..3, of every block.
// Softmax in log2 units, p = exp2(s * scale_key - m_query), masked keys
// entering exp2 as -inf (no branches). The shift m is the
// Cauchy-Schwarz bound |q| log2(e)/sqrt(d) >= every logit of the query (keys are
// unit vectors), so no max pass is needed; if a bound exceeds 60 (a query norm
// far outside the usual range) the wave takes the true row max instead, so
// exp2 never under- or overflows. Masked keys (causal: later original position;
// self) get p = 0. A query whose p are all 0 saw nothing but itself: its
// logsumexp is -1e5, as in the definition, and its output for the round (v_i)
// is not written here; the round combination reads v_i for such rounds.
// O^T = V^T P^T over 32-key steps: the B operand (P^T) comes straight from the
// S^T accumulators of two consecutive 16-key blocks (k = 8(l/16) + j: j < 4
// from the first block, j >= 4 from the second), and the A operand (V^T) from
// two 8-byte Vq reads of the same keys. In the output, lane l holds dims
// 16t + 4(l/16) + 0..3 of query l%16 for tile t, so each store writes 8 (fp16)
// or 16 (fp32) contiguous bytes. An MFMA against a block of ones gives the row
// sums of the bf16-rounded P, so numerator and denominator use the same
// weights; the logsumexp takes the fp32 sum of the unrounded p.
//
// Two variant readings run in this kernel as template flags (same overview
// page, section 2.1): NQ, queries unit-normalised too (logits scaled by 1/|q|,
// so the shift becomes log2(e)/sqrt(d); a zero query has logits 0); SB, only
// keys in the query's own bucket of the round are attendable (bucket ids
// staged per key, read through the permutation like the rows). The
// look-ahead window and the de-duplicated union have their own kernel.
#include <type_traits>

#include "dtype.h"
#include "internal.h"
#include "walks.h"

namespace lsh {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;
constexpr int kThreads = 256;  // 4 waves
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kBoundLimit = 60.0f;

template <int D>
struct Lds {
  static constexpr int kRow = D * 2 + 16;     // bytes per staged qk row
  static constexpr int kBlk8 = 8 * 16 + 16;  // bytes per 8 dims of a key pair (+16 pad)
  static constexpr int kPair = D / 8 * kBlk8;  // bytes per key pair (8 keys x d dims)
  static constexpr int kKt = 0;
  static constexpr int kVp = kKt + 2 * kChunk * kRow;
  static constexpr int kScale = kVp + 2 * (kChunk / 8) * kPair;
  static constexpr int kPos = kScale + 2 * kChunk * 4;
  static constexpr int kBound = kPos + 2 * kChunk * 4;
  static constexpr int kPermNext = kBound + 2 * kChunk * 4;  // positions of the next chunk
  static constexpr int kBkt = kPermNext + kChunk * 4;         // bucket id per key (SB)
  static constexpr int kBytes = kBkt + 2 * kChunk * 4;
};

__device__ __forceinline__ float sat16(float x) { return fminf(fmaxf(x, -65504.0f), 65504.0f); }

// One chunk's rows in flight between the loads and the staging. Thread t
// loads 16 bytes (piece t % kSegs) of qk rows t / kSegs + kRowStep k and, for
// t < kVUsers, of the 4 v rows of group t / kSegs: each load instruction of a
// wave reads whole rows. Threads t < 64 also load the squared norm of row t.
template <int D>
struct ChunkRegs {
  static constexpr int kSegs = D / 8;                      // 16-byte pieces per row
  static constexpr int kRowStep = kThreads / kSegs;        // rows per load instruction set
  static constexpr int kQ = kChunk / kRowStep;             // qk rows per thread
  static constexpr int kVUsers = (kChunk / 4) * kSegs;     // (4-key group, piece) pairs
  static_assert(kVUsers <= kThreads, "one v group piece per thread");
  static_assert(kQ * kRowStep == kChunk, "qk rows covered");
  uint4 qk[kQ];
  uint4 v[4];
  int pos;   // original position of row t % 64
  float n2;  // squared norm of qk row t (t < 64)
  int bkt;   // bucket id of row t in the round (t < 64; same-bucket reading)
};

// permutation entries (original positions) a chunk's loads need
template <int D>
struct PermRegs {
  int pos;
  int qpos[ChunkRegs<D>::kQ];
  int vpos[4];
};

// The entries come from the chunk's 64 positions staged in LDS.
template <int D>
__device__ __forceinline__ void read_perm(PermRegs<D>& pr, const int* pn) {
  using CR = ChunkRegs<D>;
  const int t = threadIdx.x;
  pr.pos = pn[t % kChunk];
#pragma unroll
  for (int k = 0; k < CR::kQ; ++k) pr.qpos[k] = pn[t / CR::kSegs + CR::kRowStep * k];
  const int qd = (t < CR::kVUsers ? t : 0) / CR::kSegs;
  const int4 q4 = *(const int4*)(pn + qd * 4);
  pr.vpos[0] = q4.x;
  pr.vpos[1] = q4.y;
  pr.vpos[2] = q4.z;
  pr.vpos[3] = q4.w;
}

// Rows are addressed as a wave-uniform base (the segment's first row) plus a
// 32-bit byte offset per lane, every offset computed before the first load,
// so no load waits for an earlier one to release its address registers.
template <int D, bool SORTED, bool SB = false>
__device__ __forceinline__ void fetch_rows(ChunkRegs<D>& cr, const PermRegs<D>& pr, int c,
                                           const uint4* qk_rows, const uint4* v_rows,
                                           const float* knorm, int64_t row0,
                                           int64_t sorted_row0, const uint16_t* bk_seg = nullptr) {
  using CR = ChunkRegs<D>;
  constexpr uint32_t kRowBytes = D * 2;
  const int t = threadIdx.x;
  const int64_t base_row = SORTED ? sorted_row0 + c * kChunk : row0;
  const unsigned char* qb = (const unsigned char*)(qk_rows + base_row * CR::kSegs);
  const unsigned char* vb = (const unsigned char*)(v_rows + base_row * CR::kSegs);
  const int qd = t / CR::kSegs, sg = t % CR::kSegs;
  uint32_t qoff[CR::kQ], voff[4];
#pragma unroll
  for (int k = 0; k < CR::kQ; ++k)
    qoff[k] = (uint32_t)(SORTED ? qd + CR::kRowStep * k : pr.qpos[k]) * kRowBytes + sg * 16;
#pragma unroll
  for (int k = 0; k < 4; ++k)
    voff[k] = (uint32_t)(SORTED ? qd * 4 + k : pr.vpos[k]) * kRowBytes + sg * 16;
  cr.pos = pr.pos;
  __builtin_amdgcn_sched_barrier(0);
  if (t < kChunk) cr.n2 = knorm[row0 + pr.pos];
  if constexpr (SB) {
    if (t < kChunk) cr.bkt = bk_seg[pr.pos];
  }
#pragma unroll
  for (int k = 0; k < CR::kQ; ++k) cr.qk[k] = *(const uint4*)(qb + qoff[k]);
  if (t < CR::kVUsers) {
#pragma unroll
    for (int k = 0; k < 4; ++k) cr.v[k] = *(const uint4*)(vb + voff[k]);
  }
}

template <int D, bool SB = false>
__device__ __forceinline__ void stage_chunk(unsigned char* lds, int sl, const ChunkRegs<D>& cr) {
  using Lay = Lds<D>;
  using CR = ChunkRegs<D>;
  const int t = threadIdx.x;
  {
    const int qd = t / CR::kSegs, sg = t % CR::kSegs;
    // (each piece passes through a register-only asm statement, so the copy
    // cannot become a memcpy from a stack copy of the registers)
#pragma unroll
    for (int k = 0; k < CR::kQ; ++k) {
      uint4 x = cr.qk[k];
      asm volatile("" : "+v"(x.x), "+v"(x.y), "+v"(x.z), "+v"(x.w));
      *(uint4*)(lds + Lay::kKt + (sl * kChunk + qd + CR::kRowStep * k) * Lay::kRow + sg * 16) = x;
    }
    if (t < kChunk) {
      const float nn = cr.n2;
      const float nrm = sqrtf(nn);
      const float sc = kLog2e / sqrtf((float)D);
      ((float*)(lds + Lay::kScale))[sl * kChunk + t] = nn > 0.f ? sc / nrm : 0.f;
      ((int*)(lds + Lay::kPos))[sl * kChunk + t] = cr.pos;
      ((float*)(lds + Lay::kBound))[sl * kChunk + t] = sc * nrm;
      if constexpr (SB) ((int*)(lds + Lay::kBkt))[sl * kChunk + t] = cr.bkt;
    }
  }
  // v rows, 4 keys x 8 dims per piece: group qd is half (qd / 4) % 2 of key
  // pair (qd % 4) + 4 (qd / 8), stored as [pair][dim][8 keys]
  if (t < CR::kVUsers) {
    const int qd = t / CR::kSegs, sg = t % CR::kSegs;
    const int pair = (qd & 3) + 4 * (qd >> 3), half = (qd >> 2) & 1;
    unsigned char* dst =
        lds + Lay::kVp + (sl * (kChunk / 8) + pair) * Lay::kPair + sg * Lay::kBlk8 + half * 8;
    const uint32_t w0[4] = {cr.v[0].x, cr.v[0].y, cr.v[0].z, cr.v[0].w};
    const uint32_t w1[4] = {cr.v[1].x, cr.v[1].y, cr.v[1].z, cr.v[1].w};
    const uint32_t w2[4] = {cr.v[2].x, cr.v[2].y, cr.v[2].z, cr.v[2].w};
    const uint32_t w3[4] = {cr.v[3].x, cr.v[3].y, cr.v[3].z, cr.v[3].w};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      *(uint2*)(dst + 32 * u) =
          make_uint2((w0[u] & 0xFFFFu) | (w1[u] << 16), (w2[u] & 0xFFFFu) | (w3[u] << 16));
      *(uint2*)(dst + 32 * u + 16) = make_uint2((w0[u] >> 16) | (w1[u] & 0xFFFF0000u),
                                                (w2[u] >> 16) | (w3[u] & 0xFFFF0000u));
    }
  }
}

// 4 consecutive fp32 outputs
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *(float4*)p = make_float4(a, b, c, d);
}

// LDS allows two workgroups (8 waves) per CU at d = 128, so each wave may take
// half the register file; say so, or the compiler aims for more waves.
// DOT (the backward's recomputation): instead of the round's rows, o receives
// per query the scalar dout(i) . o_r(i) ([seg, L] fp32; dout(i) . v_i for a
// query that saw only itself, whose output is v_i), dout being bf16 rows
// [B*H, L, D].
template <int D, typename OT, bool CAUSAL, bool SORTED, bool DOT = false, bool NQ = false,
          bool SB = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attend_mfma(
    const uint4* __restrict__ qk, const uint4* __restrict__ v, const uint4* __restrict__ qk_s,
    const uint4* __restrict__ v_s, const int32_t* __restrict__ perm,
    const float* __restrict__ knorm, OT* __restrict__ o, float* __restrict__ lse, int L, int R,
    int nseg, int chunks_per_wg, int ranges, int group_segs, int64_t o_seg_rows,
    const unsigned char* __restrict__ dout, const uint16_t* __restrict__ buckets) {
  using Lay = Lds<D>;
  constexpr int KS = D / 32;  // 32-dim K-steps of QK^T
  constexpr int DT = D / 16;  // 16-dim tiles of the output
  extern __shared__ __align__(16) unsigned char lds[];
  const int nchunks = L / kChunk;
  // Blocks walk groups of group_segs segments (all rounds of a few heads),
  // the segments of a group interleaved, so the workgroups in flight read
  // the rows of few heads, which then stay in the memory-side cache for the
  // other rounds.
  int64_t seg;
  int range;
  walks::range_block(blockIdx.x, group_segs, ranges, nseg, seg, range);
  const int c0 = range * chunks_per_wg;
  const int c1 = min(nchunks, c0 + chunks_per_wg);
  if (c0 >= c1) return;
  const int64_t bh = seg / R;
  const int32_t* pm = perm + seg * L;
  const int64_t row0 = bh * L;
  const int64_t srow0 = seg * L;
  const uint4* qk_rows = SORTED ? qk_s : qk;
  const uint4* v_rows = SORTED ? v_s : v;
  const uint16_t* bk_seg = SB ? buckets + seg * L : nullptr;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int g = lane >> 4;     // lane group: keys / dims 4g + v of a 16-wide block
  const int lq = lane & 15;    // query of this lane within the wave's 16

  ChunkRegs<D> cr;
  PermRegs<D> pr;
  int* pn = (int*)(lds + Lay::kPermNext);
  auto perm_to_lds = [&](int c) {
    if (threadIdx.x < kChunk) pn[threadIdx.x] = pm[c * kChunk + threadIdx.x];
  };
  if (c0 > 0) {
    perm_to_lds(c0 - 1);
    __syncthreads();
    read_perm<D>(pr, pn);
    fetch_rows<D, SORTED, SB>(cr, pr, c0 - 1, qk_rows, v_rows, knorm, row0, srow0, bk_seg);
    stage_chunk<D, SB>(lds, (c0 - 1) & 1, cr);
    __syncthreads();
  } else {
    // chunk 0 has no previous chunk: zero keys and values in its slot
    uint4* kt = (uint4*)(lds + Lay::kKt + kChunk * Lay::kRow);        // slot 1
    for (int i = threadIdx.x; i < kChunk * Lay::kRow / 16; i += kThreads) kt[i] = uint4{};
    uint4* vp = (uint4*)(lds + Lay::kVp + (kChunk / 8) * Lay::kPair);  // slot 1
    for (int i = threadIdx.x; i < (kChunk / 8) * Lay::kPair / 16; i += kThreads) vp[i] = uint4{};
    if (threadIdx.x < kChunk) ((float*)(lds + Lay::kScale))[kChunk + threadIdx.x] = 0.f;
  }
  perm_to_lds(c0);
  __syncthreads();
  read_perm<D>(pr, pn);
  fetch_rows<D, SORTED, SB>(cr, pr, c0, qk_rows, v_rows, knorm, row0, srow0, bk_seg);
  stage_chunk<D, SB>(lds, c0 & 1, cr);
  __syncthreads();
  if (c0 + 1 < c1) perm_to_lds(c0 + 1);
  __syncthreads();
  int pnext = 0;

  const float* kscale = (const float*)(lds + Lay::kScale);
  const int* kpos = (const int*)(lds + Lay::kPos);
  const float* kbound = (const float*)(lds + Lay::kBound);
  const int* kbkt = (const int*)(lds + Lay::kBkt);
  const uint32_t one2 = 0x3F803F80u;  // two bf16 ones
  const uint32_t ones_u[4] = {one2, one2, one2, one2};
  const bf16x8_t ones = *(const bf16x8_t*)ones_u;

  for (int c = c0; c < c1; ++c) {
    if (c + 1 < c1) {
      read_perm<D>(pr, pn);
      fetch_rows<D, SORTED, SB>(cr, pr, c + 1, qk_rows, v_rows, knorm, row0, srow0, bk_seg);
      if (c + 2 < c1 && threadIdx.x < kChunk) pnext = pm[(c + 2) * kChunk + threadIdx.x];
    }
    const int cur = c & 1, prv = cur ^ 1;
    const int kb0 = c > 0 ? 0 : 4;  // chunk 0: the first four 16-key blocks are absent
    const int q = 16 * w + lq;
    float mq = kbound[cur * kChunk + q];
    const int posq = kpos[cur * kChunk + q];
    // NQ: logits times 1/|q| (mq = log2(e)|q|/sqrt(d), so |q| = mq / that
    // factor); the Cauchy-Schwarz shift is then log2(e)/sqrt(d), or 0 for a
    // zero query (whose logits are 0)
    float qs = 1.0f;
    if constexpr (NQ) {
      const float sc = kLog2e / sqrtf((float)D);
      qs = mq > 0.f ? sc / mq : 0.f;
      mq = mq > 0.f ? sc : 0.f;
    }
    const int bq = SB ? kbkt[cur * kChunk + q] : 0;
    // DOT: the query's dout, dims 16 dt + 4g + 0..3 (as the output tiles)
    uint2 dz[DOT ? DT : 1];
    if constexpr (DOT) {
      const unsigned char* drow = dout + ((row0 + posq) * D + 4 * g) * 2;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) dz[dt] = *(const uint2*)(drow + 32 * dt);
    }
    bf16x8_t qf[KS];
    {
      const unsigned char* row = lds + Lay::kKt + (cur * kChunk + q) * Lay::kRow;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qf[ks] = *(const bf16x8_t*)(row + (32 * ks + 8 * g) * 2);
    }
    auto qk_block = [&](int kb) -> floatx4_t {
      const int sl = kb < 4 ? prv : cur;
      const unsigned char* row = lds + Lay::kKt + (sl * kChunk + (kb & 3) * 16 + lq) * Lay::kRow;
      floatx4_t acc;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8_t a = *(const bf16x8_t*)(row + (32 * ks + 8 * g) * 2);
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[ks], ks == 0 ? floatx4_t{} : acc,
                                                       0, 0, 0);
      }
      return acc;
    };
    // (absent is uniform; a bitwise or keeps it from becoming a branch that
    // splits the key reads)
    auto masked = [&](bool absent, int kp, int kbk) -> bool {
      return absent | (CAUSAL ? kp >= posq : kp == posq) | (SB && kbk != bq);
    };
    if (__ballot(mq > kBoundLimit) != 0ull) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 8; ++kb) {
        const floatx4_t sb = qk_block(kb);
        const int sl = kb < 4 ? prv : cur;
        const int key = (kb & 3) * 16 + 4 * g;
        const float4 sc = *(const float4*)(kscale + sl * kChunk + key);
        const int4 kp = *(const int4*)(kpos + sl * kChunk + key);
        const int4 kk = SB ? *(const int4*)(kbkt + sl * kChunk + key) : int4{};
        const float scv[4] = {sc.x * qs, sc.y * qs, sc.z * qs, sc.w * qs};
        const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
        const int kbv[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
        for (int b = 0; b < 4; ++b)
          mx = fmaxf(mx, masked(kb < kb0, kpv[b], kbv[b]) ? -INFINITY : sb[b] * scv[b]);
      }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      mq = mx == -INFINITY ? 0.f : mx;
    }
    float rowsum = 0.f;
    // p of the 16-key blocks 2e and 2e + 1 as the B operand of PV step e
    auto soft_pair = [&](int e, const floatx4_t& sa, const floatx4_t& sb) -> bf16x8_t {
      bf16x8_t pf;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int kb = 2 * e + half;
        const floatx4_t& s = half ? sb : sa;
        const int sl = kb < 4 ? prv : cur;
        const int key = (kb & 3) * 16 + 4 * g;
        const float4 sc = *(const float4*)(kscale + sl * kChunk + key);
        const int4 kp = *(const int4*)(kpos + sl * kChunk + key);
        const int4 kk = SB ? *(const int4*)(kbkt + sl * kChunk + key) : int4{};
        const float scv[4] = {sc.x * qs, sc.y * qs, sc.z * qs, sc.w * qs};
        const int kpv[4] = {kp.x, kp.y, kp.z, kp.w};
        const int kbv[4] = {kk.x, kk.y, kk.z, kk.w};
        const bool absent = kb < kb0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const float x = fmaf(s[b], scv[b], -mq);
          const float pv = __builtin_amdgcn_exp2f(masked(absent, kpv[b], kbv[b]) ? -INFINITY : x);
          rowsum += pv;
          pf[4 * half + b] = (__bf16)pv;
        }
      }
      return pf;
    };
    floatx4_t oacc[DT];
    floatx4_t lacc = floatx4_t{};
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) oacc[dt] = floatx4_t{};
    auto pv_step = [&](int e, const bf16x8_t& pf) {
      const int sl = e < 2 ? prv : cur;
      // key pair g + 4 (e % 2): groups 8 (e % 2) + g and 8 (e % 2) + g + 4
      const unsigned char* vp = lds + Lay::kVp + (sl * (kChunk / 8) + g + 4 * (e & 1)) * Lay::kPair +
                                (lq >> 3) * Lay::kBlk8 + (lq & 7) * 16;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8_t a = *(const bf16x8_t*)(vp + dt * 2 * Lay::kBlk8);  // dim 16 dt + lq
        oacc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pf, oacc[dt], 0, 0, 0);
      }
      lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lacc, 0, 0, 0);
    };
    // software pipeline over the four 32-key steps
    {
      floatx4_t s0 = qk_block(0), s1 = qk_block(1);
      floatx4_t s2 = qk_block(2), s3 = qk_block(3);
      const bf16x8_t p0 = soft_pair(0, s0, s1);
      floatx4_t s4 = qk_block(4), s5 = qk_block(5);
      const bf16x8_t p1 = soft_pair(1, s2, s3);
      pv_step(0, p0);
      floatx4_t s6 = qk_block(6), s7 = qk_block(7);
      const bf16x8_t p2 = soft_pair(2, s4, s5);
      pv_step(1, p1);
      const bf16x8_t p3 = soft_pair(3, s6, s7);
      pv_step(2, p2);
      pv_step(3, p3);
    }
    rowsum += __shfl_xor(rowsum, 16);
    rowsum += __shfl_xor(rowsum, 32);
    __syncthreads();  // every wave is done with slot prv
    if (c + 1 < c1) {
      stage_chunk<D, SB>(lds, prv, cr);
      if (c + 2 < c1 && threadIdx.x < kChunk) pn[threadIdx.x] = pnext;
    }
    // normalise and scatter to the query's original position: lane holds dims
    // 16t + 4g + 0..3. A query that saw only itself (l == 0) stores zeros (its
    // accumulators are 0); the round combination takes v_i for it.
    {
      const float l = lacc[0];
      const bool seen = l > 0.f;
      const float inv = seen ? 1.0f / l : 0.f;
      OT* orow = o + (seg * o_seg_rows + posq) * D;
      if constexpr (DOT) {
        float d = 0.f;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          d = fmaf(oacc[dt][0], __uint_as_float(dz[dt].x << 16), d);
          d = fmaf(oacc[dt][1], __uint_as_float(dz[dt].x & 0xFFFF0000u), d);
          d = fmaf(oacc[dt][2], __uint_as_float(dz[dt].y << 16), d);
          d = fmaf(oacc[dt][3], __uint_as_float(dz[dt].y & 0xFFFF0000u), d);
        }
        d *= inv;
        if (!seen) {  // the round's output is v_i itself
          const unsigned char* vrow = (const unsigned char*)v + ((row0 + posq) * D + 4 * g) * 2;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            const uint2 x = *(const uint2*)(vrow + 32 * dt);
            d = fmaf(__uint_as_float(x.x << 16), __uint_as_float(dz[dt].x << 16), d);
            d = fmaf(__uint_as_float(x.x & 0xFFFF0000u), __uint_as_float(dz[dt].x & 0xFFFF0000u), d);
            d = fmaf(__uint_as_float(x.y << 16), __uint_as_float(dz[dt].y << 16), d);
            d = fmaf(__uint_as_float(x.y & 0xFFFF0000u), __uint_as_float(dz[dt].y & 0xFFFF0000u), d);
          }
        }
        d += __shfl_xor(d, 16);
        d += __shfl_xor(d, 32);
        if (g == 0) o[seg * L + posq] = d;
      } else if constexpr (sizeof(OT) == 2) {
        // fp16: tiles t and t + 1 packed as 2 words per lane, then one swap of
        // odd and even 16-lane rows leaves lane group g with 8 consecutive
        // dims, 16(t + g%2) + 8(g/2) + 0..7, one 16-byte store per tile pair
        uint32_t pk[DT][2];
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
          const f16x2_t lo = {(_Float16)sat16(oacc[dt][0] * inv), (_Float16)sat16(oacc[dt][1] * inv)};
          const f16x2_t hi = {(_Float16)sat16(oacc[dt][2] * inv), (_Float16)sat16(oacc[dt][3] * inv)};
          pk[dt][0] = __builtin_bit_cast(uint32_t, lo);
          pk[dt][1] = __builtin_bit_cast(uint32_t, hi);
        }
        uint4 st[DT / 2];
#pragma unroll
        for (int j = 0; j < DT / 2; ++j) {
          const auto r0 = __builtin_amdgcn_permlane16_swap(pk[2 * j][0], pk[2 * j + 1][0], false, false);
          const auto r1 = __builtin_amdgcn_permlane16_swap(pk[2 * j][1], pk[2 * j + 1][1], false, false);
          // even g: words of tile 2j from lanes g, g + 1; odd g: tile 2j + 1
          // from lanes g - 1, g
          st[j] = make_uint4(r0[0], r1[0], r0[1], r1[1]);
        }
#pragma unroll
        for (int j = 0; j < DT / 2; ++j)
          *(uint4*)(orow + 32 * j + 16 * (g & 1) + 8 * (g >> 1)) = st[j];
      } else {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
          store4(orow + dt * 16 + 4 * g, oacc[dt][0] * inv, oacc[dt][1] * inv, oacc[dt][2] * inv,
                 oacc[dt][3] * inv);
      }
      if (g == 0) lse[seg * L + posq] = seen ? (mq + __log2f(rowsum)) * kLn2 : kSelfLogit;
    }
    __syncthreads();
  }
}

// Chunks per workgroup, and workgroups in flight the grid order is shaped for
// (two per CU on 256 CUs).
constexpr int kRangeChunks = 16;
constexpr int kResidentBlocks = 512;

template <int D, typename OT, bool CAUSAL, bool SORTED, bool DOT = false, bool NQ = false,
          bool SB = false>
void launch_one(const Problem& p, const void* qk, const void* v, const void* qk_s,
                const void* v_s, const int32_t* perm, const float* knorm, OT* o, float* lse,
                hipStream_t s, const void* dout = nullptr, const uint16_t* buckets = nullptr) {
  const int64_t nseg = p.nseg();
  // whole heads (all their rounds) per group, enough to fill the resident set
  const walks::RangeShape sh =
      walks::range_shape(p.L / kChunk, nseg, p.R, kRangeChunks, kResidentBlocks);
  const size_t shmem = Lds<D>::kBytes;
  hipLaunchKernelGGL((k_attend_mfma<D, OT, CAUSAL, SORTED, DOT, NQ, SB>), dim3((unsigned)sh.blocks),
                     dim3(kThreads), shmem, s, (const uint4*)qk, (const uint4*)v,
                     (const uint4*)qk_s, (const uint4*)v_s, perm, knorm, o, lse, p.L, p.R,
                     (int)nseg, sh.per, sh.ranges, sh.group_segs, p.o_seg_rows(),
                     (const unsigned char*)dout, buckets);
}

// the unit-query and same-bucket readings (fused gather only)
template <int D, typename OT, bool CAUSAL>
void launch_nq_sb(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                  const float* knorm, const uint16_t* buckets, OT* o, float* lse, hipStream_t s) {
  const bool nq = (p.flags & LSH_ATTN_FLAG_NORM_QUERIES) != 0;
  const bool sb = (p.flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  if (nq && sb)
    launch_one<D, OT, CAUSAL, false, false, true, true>(p, qk, v, nullptr, nullptr, perm, knorm,
                                                        o, lse, s, nullptr, buckets);
  else if (nq)
    launch_one<D, OT, CAUSAL, false, false, true, false>(p, qk, v, nullptr, nullptr, perm, knorm,
                                                         o, lse, s, nullptr, buckets);
  else
    launch_one<D, OT, CAUSAL, false, false, false, true>(p, qk, v, nullptr, nullptr, perm, knorm,
                                                         o, lse, s, nullptr, buckets);
}

template <int D, typename OT>
void launch_d(const Problem& p, const void* qk, const void* v, const void* qk_s, const void* v_s,
              const int32_t* perm, const float* knorm, const uint16_t* buckets, OT* o,
              float* lse, hipStream_t s) {
  if (p.flags & (LSH_ATTN_FLAG_NORM_QUERIES | LSH_ATTN_FLAG_SAME_BUCKET)) {
    if (p.causal) launch_nq_sb<D, OT, true>(p, qk, v, perm, knorm, buckets, o, lse, s);
    else launch_nq_sb<D, OT, false>(p, qk, v, perm, knorm, buckets, o, lse, s);
    return;
  }
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
  // unit queries and the same-bucket mask run here too (with the gather fused);
  // the look-ahead window and the de-duplicated union have their own kernel
  const int own = LSH_ATTN_FLAG_LOOK_AHEAD | LSH_ATTN_FLAG_DEDUP;
  const int here = LSH_ATTN_FLAG_NORM_QUERIES | LSH_ATTN_FLAG_SAME_BUCKET;
  return p.dtype == LSH_ATTN_BF16 && p.m == kChunk && (p.d == 64 || p.d == 128) &&
         !(p.flags & own) &&
         (!(p.flags & here) || !(p.flags & LSH_ATTN_FLAG_SEPARATE_GATHER));
}

template <typename OT>
hipError_t launch_attend_mfma(const Problem& p, const void* qk, const void* v,
                              const void* qk_sorted, const void* v_sorted, const int32_t* perm,
                              const float* knorm, const uint16_t* buckets, OT* o, float* lse,
                              hipStream_t s) {
  static bool configured[kMaxDevices] = {};
  if (first_on_device(configured)) {
    // allow the dynamic LDS size above the 64 KiB default
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, true, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, false, false>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, true, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    (void)hipFuncSetAttribute((const void*)k_attend_mfma<128, OT, false, true>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
    const void* variants[] = {
        (const void*)k_attend_mfma<128, OT, true, false, false, true, false>,
        (const void*)k_attend_mfma<128, OT, true, false, false, false, true>,
        (const void*)k_attend_mfma<128, OT, true, false, false, true, true>,
        (const void*)k_attend_mfma<128, OT, false, false, false, true, false>,
        (const void*)k_attend_mfma<128, OT, false, false, false, false, true>,
        (const void*)k_attend_mfma<128, OT, false, false, false, true, true>};
    for (const void* f : variants)
      (void)hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, Lds<128>::kBytes);
  }
  if (p.d == 64) launch_d<64, OT>(p, qk, v, qk_sorted, v_sorted, perm, knorm, buckets, o, lse, s);
  else launch_d<128, OT>(p, qk, v, qk_sorted, v_sorted, perm, knorm, buckets, o, lse, s);
  return hipGetLastError();
}

hipError_t launch_attend_mfma_dot(const Problem& p, const void* qk, const void* v,
                                  const int32_t* perm, const float* knorm, const void* dout,
                                  const uint16_t* buckets, float* od, float* lse, hipStream_t s) {
  static bool configured[kMaxDevices] = {};
  if (first_on_device(configured)) {
    auto attr = [](const void* k) {
      (void)hipFuncSetAttribute(k, hipFuncAttributeMaxDynamicSharedMemorySize,
                                Lds<128>::kBytes);
    };
    attr((const void*)k_attend_mfma<128, float, true, false, true>);
    attr((const void*)k_attend_mfma<128, float, false, false, true>);
    attr((const void*)k_attend_mfma<128, float, true, false, true, true, false>);
    attr((const void*)k_attend_mfma<128, float, false, false, true, true, false>);
    attr((const void*)k_attend_mfma<128, float, true, false, true, false, true>);
    attr((const void*)k_attend_mfma<128, float, false, false, true, false, true>);
    attr((const void*)k_attend_mfma<128, float, true, false, true, true, true>);
    attr((const void*)k_attend_mfma<128, float, false, false, true, true, true>);
  }
  // the unit-query and same-bucket readings as in the forward (template flags)
  const bool nq = (p.flags & LSH_ATTN_FLAG_NORM_QUERIES) != 0;
  const bool sb = (p.flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  auto go = [&](auto d, auto c, auto n, auto b) {
    constexpr int D = decltype(d)::value;
    constexpr bool C = decltype(c)::value, NQ = decltype(n)::value, SB = decltype(b)::value;
    launch_one<D, float, C, false, true, NQ, SB>(p, qk, v, nullptr, nullptr, perm, knorm, od, lse,
                                                 s, dout, buckets);
  };
  auto flags = [&](auto d, auto c) {
    using T = std::true_type;
    using F = std::false_type;
    if (nq && sb) go(d, c, T{}, T{});
    else if (nq) go(d, c, T{}, F{});
    else if (sb) go(d, c, F{}, T{});
    else go(d, c, F{}, F{});
  };
  auto causal = [&](auto d) {
    if (p.causal) flags(d, std::true_type{});
    else flags(d, std::false_type{});
  };
  if (p.d == 64) causal(std::integral_constant<int, 64>{});
  else causal(std::integral_constant<int, 128>{});
  return hipGetLastError();
}

template hipError_t launch_attend_mfma<float>(const Problem&, const void*, const void*, const void*,
                                              const void*, const int32_t*, const float*,
                                              const uint16_t*, float*, float*, hipStream_t);
template hipError_t launch_attend_mfma<_Float16>(const Problem&, const void*, const void*,
                                                 const void*, const void*, const int32_t*,
                                                 const float*, const uint16_t*, _Float16*, float*,
                                                 hipStream_t);

}  // namespace lsh
