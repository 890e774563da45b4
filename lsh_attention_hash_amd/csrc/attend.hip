// attend.hip -- chunked look-one-back attention over the sorted sequence.
//
// Reformer summary (p2.ttnews.xyz), section on LSH attention: the sorted
// sequence is cut into chunks of m and attention stays inside a chunk; the
// Reformer overview (www.dtcms.com/a/488796.html, section 2.1) lets a query
// also see the neighbouring chunk; taken here as the chunk itself plus the
// previous one (chunk 0 has no look-back). Keys are unit-normalised (same
// section), logits are scaled by 1/sqrt(d) (its softmax formula). The causal
// mask compares original positions. Self-mask (first page, shared-QK
// section): the query's own key gets logit -1e5, so it carries weight only
// when nothing else is attendable; then o = v_i and lse = -1e5 exactly.
//
// This is the plain kernel (fp32 rows, chunk lengths other than 64, and the
// variant combinations the matrix-core kernels do not take): an online
// softmax in fp32 over the window's keys. Per-round results are written at
// the ORIGINAL position (this is the unsort).
//
// Variant readings (flags): LOOK_AHEAD adds the next chunk
// to the window; SAME_BUCKET keeps only keys in the query's bucket of the
// round; NORM_QUERIES unit-normalises the query; DEDUP lowers each logit by
// log N_ij, N_ij being the number of rounds whose window gives key j to query
// i (window membership from each round's inverse permutation, with the same
// bucket test), so that the combination is one softmax over the union of the
// rounds' key sets, each key once.
#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

// DEDUP: the number of rounds of head bh whose window holds key j for query
// i (self and causal masks do not depend on the round)
__device__ __forceinline__ int rounds_sharing(const int32_t* __restrict__ inv,
                                              const uint16_t* __restrict__ bkt, int64_t bh,
                                              int L, int m, int R, int flags, int i, int j) {
  int n = 0;
  for (int r = 0; r < R; ++r) {
    const int64_t base = (bh * R + r) * L;
    const int ci = inv[base + i] / m, cj = inv[base + j] / m;
    bool in = cj == ci || cj == ci - 1 || ((flags & LSH_ATTN_FLAG_LOOK_AHEAD) && cj == ci + 1);
    if (flags & LSH_ATTN_FLAG_SAME_BUCKET) in = in && bkt[base + j] == bkt[base + i];
    n += in ? 1 : 0;
  }
  return n;
}

// One workgroup of 256 threads per (segment, chunk, block of kQB queries).
// The window's permutation entries (and bucket ids) are read into LDS first;
// its keys are then taken kKB at a time: their qk and v rows are staged in LDS
// as fp32 with coalesced 16-byte loads, the next block's rows being loaded
// into registers while the current one is computed. Thread t serves query
// t / 16 of the block: the logits of keys (t % 16) + 16 u, an online softmax
// whose running max and sum the 16 threads of a query share (the block's max
// and sum reduced over them), then output dims (t % 16) kDPT .. + kDPT.
template <int D>
struct Simple {
  static constexpr int kQB = 16;                   // queries per workgroup
  static constexpr int kKB = D == 64 ? 64 : 32;    // keys per staged block
  static constexpr int kKPT = kKB / 16;            // logits per thread
  static constexpr int kDPT = D / 16;              // output dims per thread
  static constexpr int kS = D + 4;                 // LDS row stride (fp32 words)
  static constexpr int kPieces = kKB * D / 4 / 256;  // 4-element loads per thread per array
  static constexpr int kTPK = 256 / kKB;           // threads per key in the norm pass
  static constexpr int kMaxWin = 3 * 256;          // window slots (chunk_len <= 256)
};

// four consecutive elements of a row as fp32
__device__ __forceinline__ float4 load4(const float* p) { return *(const float4*)p; }
__device__ __forceinline__ float4 load4(const bf16_t* p) {
  const uint2 u = *(const uint2*)p;
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xFFFF0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xFFFF0000u));
}

template <int D, typename T>
__global__ __launch_bounds__(256) void k_attend_simple(
    const T* __restrict__ qk, const T* __restrict__ v, const T* __restrict__ qk_s,
    const T* __restrict__ v_s, const int32_t* __restrict__ perm, float* __restrict__ o,
    float* __restrict__ lse, int L, int m, int R, int causal, int64_t o_seg_rows, int flags,
    const uint16_t* __restrict__ bkt, const int32_t* __restrict__ inv) {
  using S = Simple<D>;
  __shared__ __align__(16) float ks[S::kKB * S::kS];
  __shared__ __align__(16) float vs[S::kKB * S::kS];
  __shared__ __align__(16) float qs[S::kQB * S::kS];
  __shared__ float ps[S::kQB * S::kKB];
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
  const bool sorted = qk_s != nullptr;
  const bool same_bucket = (flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  const int first = (c > 0 ? c - 1 : c) * m;
  int last = (c + 1) * m;
  if ((flags & LSH_ATTN_FLAG_LOOK_AHEAD) && last < L) last += m;
  const int nwin = last - first;
  for (int x = tid; x < nwin; x += 256) {
    const int j = pm[first + x];
    pw[x] = j;
    if (same_bucket) bw[x] = bkt[seg * L + j];
  }
  __syncthreads();

  // the block's queries (slot c m + qb kQB + ql), rows staged as fp32
  const int q = tid / 16, g = tid % 16;
  const int qslot0 = c * m + qb * S::kQB;
  const int nq = min(S::kQB, (c + 1) * m - qslot0);
  for (int p = tid; p < S::kQB * D / 4; p += 256) {
    const int ql = p / (D / 4), col = (p % (D / 4)) * 4;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (ql < nq) {
      const int sl = qslot0 + ql;
      const T* row = sorted ? qk_s + (seg * L + sl) * D : qk + (bh * L + pw[sl - first]) * D;
      x = load4(row + col);
    }
    *(float4*)&qs[ql * S::kS + col] = x;
  }
  const bool active = q < nq;
  const int i = active ? pw[qslot0 + q - first] : 0;
  const int bi = same_bucket && active ? bw[qslot0 + q - first] : 0;
  __syncthreads();
  if (flags & LSH_ATTN_FLAG_NORM_QUERIES) {
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

  // rows of key block kb -> registers (kPieces 4-element pieces per array)
  float4 kr[S::kPieces], vr[S::kPieces];
  auto fetch = [&](int kb) {
    const int t0 = kb * S::kKB;
#pragma unroll
    for (int u = 0; u < S::kPieces; ++u) {
      const int p = tid + 256 * u;
      const int kk = p / (D / 4), col = (p % (D / 4)) * 4;
      const int x = t0 + kk;
      if (x < nwin) {
        const int64_t row = sorted ? (seg * L + first + x) * D : (bh * L + pw[x]) * D;
        kr[u] = load4((sorted ? qk_s : qk) + row + col);
        vr[u] = load4((sorted ? v_s : v) + row + col);
      } else {
        kr[u] = make_float4(0.f, 0.f, 0.f, 0.f);
        vr[u] = kr[u];
      }
    }
  };
  const float scale = 1.0f / sqrtf((float)D);
  const bool dedup = (flags & LSH_ATTN_FLAG_DEDUP) != 0;
  float mx = -INFINITY, l = 0.f;
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
    {  // squared key norms: kTPK threads per key, D / kTPK elements each
      const int kk = tid / S::kTPK, part = tid % S::kTPK;
      float nn = 0.f;
#pragma unroll
      for (int u = 0; u < D / S::kTPK; ++u) {
        const float x = ks[kk * S::kS + part * (D / S::kTPK) + u];
        nn += x * x;
      }
#pragma unroll
      for (int off = 1; off < S::kTPK; off <<= 1) nn += __shfl_xor(nn, off);
      if (part == 0) nrm[kk] = nn;
    }
    __syncthreads();
    // logits of keys g + 16 u
    float sv[S::kKPT];
    float bmax = -INFINITY;
#pragma unroll
    for (int u = 0; u < S::kKPT; ++u) {
      const int kk = g + 16 * u;
      sv[u] = -INFINITY;
      if (active && kk < nk) {
        const int j = pw[t0 + kk];
        bool keep = !(causal && j > i);
        if (same_bucket && j != i && bw[t0 + kk] != bi) keep = false;
        if (keep) {
          float dot = 0.f;
#pragma unroll
          for (int col = 0; col < D; col += 4) {
            const float4 a = *(const float4*)&qs[q * S::kS + col];
            const float4 b = *(const float4*)&ks[kk * S::kS + col];
            dot = fmaf(a.x, b.x, dot);
            dot = fmaf(a.y, b.y, dot);
            dot = fmaf(a.z, b.z, dot);
            dot = fmaf(a.w, b.w, dot);
          }
          const float nn = nrm[kk];
          float logit = (j == i) ? kSelfLogit : (nn > 0.f ? dot / sqrtf(nn) * scale : 0.f);
          if (dedup && j != i)
            logit -= __logf((float)rounds_sharing(inv, bkt, bh, L, m, R, flags, i, j));
          sv[u] = logit;
          bmax = fmaxf(bmax, logit);
        }
      }
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) bmax = fmaxf(bmax, __shfl_xor(bmax, off));
    const float mnew = fmaxf(mx, bmax);
    // nothing attendable yet: weights stay 0 and the running state as is
    const bool none = mnew == -INFINITY;
    const float corr = none ? 1.f : __expf(mx - mnew);
    float bsum = 0.f;
#pragma unroll
    for (int u = 0; u < S::kKPT; ++u) {
      const float pj = none ? 0.f : __expf(sv[u] - mnew);
      bsum += pj;
      ps[q * S::kKB + g + 16 * u] = pj;
    }
#pragma unroll
    for (int off = 1; off < 16; off <<= 1) bsum += __shfl_xor(bsum, off);
    l = l * corr + bsum;
    mx = mnew;
    // the 16 threads of a query (one wave) wrote ps; each now reads them all
#pragma unroll
    for (int u = 0; u < S::kDPT; ++u) acc[u] *= corr;
    for (int kk = 0; kk < nk; ++kk) {
      const float pj = ps[q * S::kKB + kk];
#pragma unroll
      for (int u = 0; u < S::kDPT; u += 4) {
        const float4 b = *(const float4*)&vs[kk * S::kS + g * S::kDPT + u];
        acc[u] = fmaf(pj, b.x, acc[u]);
        acc[u + 1] = fmaf(pj, b.y, acc[u + 1]);
        acc[u + 2] = fmaf(pj, b.z, acc[u + 2]);
        acc[u + 3] = fmaf(pj, b.w, acc[u + 3]);
      }
    }
    __syncthreads();
  }
  if (!active) return;
  float* orow = o + (seg * o_seg_rows + i) * D + g * S::kDPT;
  const float inv_l = 1.0f / l;
#pragma unroll
  for (int u = 0; u < S::kDPT; u += 4)
    *(float4*)(orow + u) =
        make_float4(acc[u] * inv_l, acc[u + 1] * inv_l, acc[u + 2] * inv_l, acc[u + 3] * inv_l);
  if (g == 0) lse[seg * L + i] = mx + logf(l);
}

template <int D, typename T>
void launch_simple(const Problem& p, const void* qk, const void* v, const void* qk_s,
                   const void* v_s, const int32_t* perm, const uint16_t* bkt, const int32_t* inv,
                   float* o, float* lse, hipStream_t s) {
  const int qblocks = (p.m + Simple<D>::kQB - 1) / Simple<D>::kQB;
  const dim3 grid((unsigned)((int64_t)(p.L / p.m) * qblocks * p.nseg()));
  hipLaunchKernelGGL((k_attend_simple<D, T>), grid, dim3(256), 0, s, (const T*)qk,
                     (const T*)v, (const T*)qk_s, (const T*)v_s, perm, o, lse, p.L, p.m, p.R,
                     p.causal, p.o_seg_rows(), p.flags & kVariantFlags, bkt, inv);
}

__global__ void k_inverse_perm(const int32_t* __restrict__ perm, int32_t* __restrict__ inv,
                               int L, int64_t n) {
  const int64_t x = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (x >= n) return;
  const int64_t seg = x / L;
  inv[seg * L + perm[x]] = (int32_t)(x - seg * L);
}

}  // namespace

hipError_t launch_attend_plain(const Problem& p, const void* qk, const void* v,
                               const int32_t* perm, const uint16_t* buckets, const int32_t* inv,
                               float* o, float* lse, hipStream_t s) {
  const bool bf = p.dtype == LSH_ATTN_BF16;
  if (p.d == 64) {
    if (bf) launch_simple<64, bf16_t>(p, qk, v, nullptr, nullptr, perm, buckets, inv, o, lse, s);
    else launch_simple<64, float>(p, qk, v, nullptr, nullptr, perm, buckets, inv, o, lse, s);
  } else if (p.d == 128) {
    if (bf) launch_simple<128, bf16_t>(p, qk, v, nullptr, nullptr, perm, buckets, inv, o, lse, s);
    else launch_simple<128, float>(p, qk, v, nullptr, nullptr, perm, buckets, inv, o, lse, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_inverse_perm(const Problem& p, const int32_t* perm, int32_t* inv, hipStream_t s) {
  const int64_t n = p.n_rows();
  hipLaunchKernelGGL(k_inverse_perm, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, perm,
                     inv, p.L, n);
  return hipGetLastError();
}

hipError_t launch_attend(const Problem& p, const void* qk, const void* v, const void* qk_sorted,
                         const void* v_sorted, const int32_t* perm, const float* knorm,
                         const uint16_t* buckets, const int32_t* inv, float* o, float* lse,
                         hipStream_t s) {
  if (attend_mfma_supported(p)) {
    if (round_outputs_half(p))
      return launch_attend_mfma<_Float16>(p, qk, v, qk_sorted, v_sorted, perm, knorm, buckets,
                                          (_Float16*)o, lse, s);
    return launch_attend_mfma<float>(p, qk, v, qk_sorted, v_sorted, perm, knorm, buckets, o, lse,
                                     s);
  }
  if (attend_variant_mfma_supported(p))
    return launch_attend_variant_mfma(p, qk, v, perm, knorm, buckets, inv, o, lse, s);
  const bool bf = p.dtype == LSH_ATTN_BF16;
  if (p.d == 64) {
    if (bf) launch_simple<64, bf16_t>(p, qk, v, qk_sorted, v_sorted, perm, buckets, inv, o, lse, s);
    else launch_simple<64, float>(p, qk, v, qk_sorted, v_sorted, perm, buckets, inv, o, lse, s);
  } else if (p.d == 128) {
    if (bf) launch_simple<128, bf16_t>(p, qk, v, qk_sorted, v_sorted, perm, buckets, inv, o, lse, s);
    else launch_simple<128, float>(p, qk, v, qk_sorted, v_sorted, perm, buckets, inv, o, lse, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace lsh
