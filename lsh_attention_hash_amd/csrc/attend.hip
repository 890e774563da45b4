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
// This is the plain kernel: one thread per query slot, an online softmax in
// fp32 over the window's keys, rows read from global memory. Per-round
// results are written at the ORIGINAL position (this is the unsort).
//
// Variant readings (flags, this kernel only): LOOK_AHEAD adds the next chunk
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

template <int D, typename T>
__global__ __launch_bounds__(256) void k_attend_simple(
    const T* __restrict__ qk, const T* __restrict__ v, const T* __restrict__ qk_s,
    const T* __restrict__ v_s, const int32_t* __restrict__ perm, float* __restrict__ o,
    float* __restrict__ lse, int L, int m, int R, int causal, int64_t o_seg_rows, int flags,
    const uint16_t* __restrict__ bkt, const int32_t* __restrict__ inv) {
  if ((int)threadIdx.x >= m) return;
  const int nchunks = L / m;
  const int64_t seg = blockIdx.x / (unsigned)nchunks;
  const int c = (int)(blockIdx.x % (unsigned)nchunks);
  const int s = c * m + threadIdx.x;
  const int64_t bh = seg / R;
  const int32_t* pm = perm + seg * L;
  const int i = pm[s];
  const bool sorted = qk_s != nullptr;
  const T* qrow = sorted ? qk_s + (seg * L + s) * D : qk + (bh * L + i) * D;
  float q[D], acc[D];
  float qq = 0.f;
#pragma unroll
  for (int u = 0; u < D; ++u) {
    q[u] = to_f32(qrow[u]);
    qq += q[u] * q[u];
    acc[u] = 0.f;
  }
  if (flags & LSH_ATTN_FLAG_NORM_QUERIES) {
    const float rq = qq > 0.f ? 1.0f / sqrtf(qq) : 0.f;
#pragma unroll
    for (int u = 0; u < D; ++u) q[u] *= rq;
  }
  const bool same_bucket = (flags & LSH_ATTN_FLAG_SAME_BUCKET) != 0;
  const int bi = same_bucket ? bkt[seg * L + i] : 0;
  const float scale = 1.0f / sqrtf((float)D);
  float mx = -INFINITY, l = 0.f;
  const int first = (c > 0 ? c - 1 : c) * m;
  int last = (c + 1) * m;
  if ((flags & LSH_ATTN_FLAG_LOOK_AHEAD) && last < L) last += m;
  for (int t = first; t < last; ++t) {
    const int j = pm[t];
    if (causal && j > i) continue;
    if (same_bucket && j != i && bkt[seg * L + j] != bi) continue;
    const T* krow = sorted ? qk_s + (seg * L + t) * D : qk + (bh * L + j) * D;
    const T* vrow = sorted ? v_s + (seg * L + t) * D : v + (bh * L + j) * D;
    float dot = 0.f, nn = 0.f;
#pragma unroll
    for (int u = 0; u < D; ++u) {
      const float kk = to_f32(krow[u]);
      dot += q[u] * kk;
      nn += kk * kk;
    }
    float logit = (j == i) ? kSelfLogit : (nn > 0.f ? dot / sqrtf(nn) * scale : 0.f);
    if ((flags & LSH_ATTN_FLAG_DEDUP) && j != i)
      logit -= __logf((float)rounds_sharing(inv, bkt, bh, L, m, R, flags, i, j));
    const float mnew = fmaxf(mx, logit);
    const float corr = __expf(mx - mnew);
    const float pj = __expf(logit - mnew);
    l = l * corr + pj;
#pragma unroll
    for (int u = 0; u < D; ++u) acc[u] = acc[u] * corr + pj * to_f32(vrow[u]);
    mx = mnew;
  }
  float* orow = o + (seg * o_seg_rows + i) * D;
  const float inv_l = 1.0f / l;
#pragma unroll
  for (int u = 0; u < D; ++u) orow[u] = acc[u] * inv_l;
  lse[seg * L + i] = mx + logf(l);
}

template <int D, typename T>
void launch_simple(const Problem& p, const void* qk, const void* v, const void* qk_s,
                   const void* v_s, const int32_t* perm, const uint16_t* bkt, const int32_t* inv,
                   float* o, float* lse, hipStream_t s) {
  const dim3 grid((unsigned)((p.L / p.m) * p.nseg()));
  const int block = ((p.m + kWave - 1) / kWave) * kWave;
  hipLaunchKernelGGL((k_attend_simple<D, T>), grid, dim3(block), 0, s, (const T*)qk,
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
