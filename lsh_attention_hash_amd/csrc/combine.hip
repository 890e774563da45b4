// combine.hip -- logsumexp-weighted combination of the hash rounds.
//
// The multi-round section of the Reformer summary (p2.ttnews.xyz) leaves the
// combination to the original paper. Reading taken: out(i) is the softmax
// over rounds of lse_r(i) applied to the per-round outputs,
//   w_r = exp(lse_r - max_r lse_r) / sum_r' exp(lse_r' - max_r lse_r'),
//   out(i) = sum_r w_r o_r(i),
// which equals one softmax over the multiset union of all rounds' windows.
// The per-round rows are already at original positions (the attention kernel
// scatters them), so this kernel streams them in order. A round whose
// logsumexp is the self-only value -1e5 has output v_i by definition; that row
// is taken from v, the round's own row (finite, zeros on the matrix-core path)
// entering with weight 0.
// fp16 per-round rows hold at most +-65504 (the attention clamps them there);
// every (position, 8 dims) piece whose rounds reached that limit is counted
// in *at_limit, so the caller can tell the result is inaccurate (and keep the
// rows in fp32).
#include <type_traits>

#include "dtype.h"
#include "internal.h"

namespace lsh {
namespace {

// 8 consecutive per-round outputs as floats. Each row is read exactly once,
// so the loads are non-temporal (streamed past the caches).
__device__ __forceinline__ void load8(const float* p, float* x, uint32_t&) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  const f32x4_t a = __builtin_nontemporal_load((const f32x4_t*)p);
  const f32x4_t b = __builtin_nontemporal_load((const f32x4_t*)(p + 4));
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    x[j] = a[j];
    x[4 + j] = b[j];
  }
}
// lim: bit 15 or 31 is set when a half-word's magnitude bits reach 0x7BFF
// (65504, the largest finite fp16) or beyond (x + 0x0401 carries into the
// sign position; no carry crosses into the other half-word)
__device__ __forceinline__ void load8(const _Float16* p, float* x, uint32_t& lim) {
  typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const f16x8_t a = __builtin_nontemporal_load((const f16x8_t*)p);
  const u32x4_t b = __builtin_bit_cast(u32x4_t, a);
#pragma unroll
  for (int j = 0; j < 4; ++j) lim |= (b[j] & 0x7FFF7FFFu) + 0x04010401u;
#pragma unroll
  for (int j = 0; j < 8; ++j) x[j] = (float)a[j];
}
// 8 consecutive inputs (v) as floats
__device__ __forceinline__ void load8(const float* p, float* x) {
  const float4 a = *(const float4*)p, b = *(const float4*)(p + 4);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}
__device__ __forceinline__ void load8(const bf16_t* p, float* x) {
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

// Each lane owns 8 consecutive dims of one row; D/8 lanes cover a row.
// kR > 0: R == kR, every round's logsumexp and row loaded before any use.
// kR == 0 (other round counts): rounds taken 4 at a time, a first pass over
// the logsumexps for the max, then the rows.
template <int D, typename OutT, typename OT, typename VT, int kR>
__global__ __launch_bounds__(256) void k_combine(const OT* __restrict__ o,
                                                 const float* __restrict__ lse,
                                                 const VT* __restrict__ v,
                                                 OutT* __restrict__ out, int L, int R_rt,
                                                 int64_t n_rows, int64_t o_seg_rows,
                                                 unsigned long long* __restrict__ at_limit) {
  constexpr int kLpr = D / 8;             // lanes per row
  constexpr int kRpb = 256 / kLpr;        // rows per block
  constexpr int kG = kR > 0 ? kR : 4;     // rounds per group
  const int R = kR > 0 ? kR : R_rt;
  const int sub = threadIdx.x % kLpr;
  const int64_t stride = (int64_t)gridDim.x * kRpb;
  // Blocks walk the rows from the end: the attention kernel finishes the last
  // heads last, so their rows are read first, while they are most likely
  // still in the memory-side cache.
  for (int64_t row = (int64_t)(gridDim.x - 1 - blockIdx.x) * kRpb + threadIdx.x / kLpr; row < n_rows;
       row += stride) {
    const int64_t bh = row / L;
    const int64_t i = row - bh * L;
    const float* lr = lse + bh * R * L + i;
    const OT* orow = o + (bh * R * o_seg_rows + i) * D + sub * 8;
    float mx = -INFINITY;
    float sum = 0.f, acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float wself = 0.f;  // weight of the self-only rounds
    uint32_t lim = 0;
    // rounds r0 .. r0 + kG - 1 given their logsumexps and rows, mx final
    auto accumulate = [&](int r0, const float* lv, float (*x)[8]) {
#pragma unroll
      for (int u = 0; u < kG; ++u) {
        const float w = __expf(lv[u] - mx);  // 0 for rounds past R
        const bool self_only = lv[u] == kSelfLogit;
        sum += w;
        wself += self_only ? w : 0.f;
        const float wo = self_only ? 0.f : w;
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] = fmaf(wo, x[u][j], acc[j]);
      }
    };
    if constexpr (kR > 0) {
      float lv[kR], x[kR][8];
#pragma unroll
      for (int u = 0; u < kR; ++u) lv[u] = lr[(int64_t)u * L];
#pragma unroll
      for (int u = 0; u < kR; ++u) load8(orow + u * o_seg_rows * D, x[u], lim);
#pragma unroll
      for (int u = 0; u < kR; ++u) mx = fmaxf(mx, lv[u]);
      accumulate(0, lv, x);
    } else {
      for (int r0 = 0; r0 < R; r0 += kG) {
        float lv[kG];
#pragma unroll
        for (int u = 0; u < kG; ++u) lv[u] = r0 + u < R ? lr[(int64_t)(r0 + u) * L] : -INFINITY;
#pragma unroll
        for (int u = 0; u < kG; ++u) mx = fmaxf(mx, lv[u]);
      }
      for (int r0 = 0; r0 < R; r0 += kG) {
        float lv[kG], x[kG][8] = {};
#pragma unroll
        for (int u = 0; u < kG; ++u) {
          const bool in = r0 + u < R;
          lv[u] = in ? lr[(int64_t)(r0 + u) * L] : -INFINITY;  // weight 0 past R
          if (in) load8(orow + (r0 + u) * o_seg_rows * D, x[u], lim);
        }
        accumulate(r0, lv, x);
      }
    }
    const float inv_sum = 1.0f / sum;
    if (wself > 0.f) {
      float x[8];
      load8(v + row * D + sub * 8, x);
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = fmaf(wself, x[j], acc[j]);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] *= inv_sum;
    store8(out + row * D + sub * 8, acc);
    if (lim & 0x80008000u) atomicAdd(at_limit, 1ull);
  }
}

template <int D, typename OT, typename VT>
void launch_t(const Problem& p, const OT* o, const float* lse, const VT* v, void* out,
              unsigned long long* at_limit, hipStream_t s) {
  const int64_t n = p.n_token_heads();
  const int64_t rpb = 256 / (D / 8);
  const int64_t want = (n + rpb - 1) / rpb;
  const unsigned blocks = (unsigned)(want < 262144 ? want : 262144);
  auto go = [&](auto g) {
    constexpr int G = decltype(g)::value;
    if (p.out_dtype == LSH_ATTN_BF16)
      hipLaunchKernelGGL((k_combine<D, bf16_t, OT, VT, G>), dim3(blocks), dim3(256), 0, s, o, lse,
                         v, (bf16_t*)out, p.L, p.R, n, p.o_seg_rows(), at_limit);
    else
      hipLaunchKernelGGL((k_combine<D, float, OT, VT, G>), dim3(blocks), dim3(256), 0, s, o, lse,
                         v, (float*)out, p.L, p.R, n, p.o_seg_rows(), at_limit);
  };
  switch (p.R) {
    case 1: go(std::integral_constant<int, 1>{}); break;
    case 2: go(std::integral_constant<int, 2>{}); break;
    case 3: go(std::integral_constant<int, 3>{}); break;
    case 4: go(std::integral_constant<int, 4>{}); break;
    case 8: go(std::integral_constant<int, 8>{}); break;
    default: go(std::integral_constant<int, 0>{}); break;
  }
}

template <int D, typename OT>
void launch_v(const Problem& p, const OT* o, const float* lse, const void* v, void* out,
              unsigned long long* at_limit, hipStream_t s) {
  if (p.dtype == LSH_ATTN_BF16)
    launch_t<D, OT, bf16_t>(p, o, lse, (const bf16_t*)v, out, at_limit, s);
  else
    launch_t<D, OT, float>(p, o, lse, (const float*)v, out, at_limit, s);
}

}  // namespace

hipError_t launch_combine(const Problem& p, const void* o, bool o_half, const float* lse,
                          const void* v, void* out, unsigned long long* at_limit,
                          hipStream_t s) {
  if (p.d == 64) {
    if (o_half) launch_v<64, _Float16>(p, (const _Float16*)o, lse, v, out, at_limit, s);
    else launch_v<64, float>(p, (const float*)o, lse, v, out, at_limit, s);
  } else {
    if (o_half) launch_v<128, _Float16>(p, (const _Float16*)o, lse, v, out, at_limit, s);
    else launch_v<128, float>(p, (const float*)o, lse, v, out, at_limit, s);
  }
  return hipGetLastError();
}

}  // namespace lsh
