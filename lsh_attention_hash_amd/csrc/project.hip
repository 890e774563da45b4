// project.hip -- the shared-QK and value projections of a layer input, feeding
// the hash.
//
// Reformer summary (p2.ttnews.xyz), shared-QK section: one linear map gives
// the queries and the keys, a second one the values:
//   qk[b, h, i, e] = sum_k x[b, i, k] w_qk[h d + e, k],   v likewise with w_v,
// x [B, L, model_dim] and the weights [H d, model_dim] (a linear layer's
// weight, model_dim -> H d features), qk and v written as [B, H, L, d] in the
// input dtype.
//
// Matrix-core path (bf16, d in {64, 128}, model_dim a multiple of 32): one
// workgroup computes a 256-row x d-column tile of one head's qk or v with the
// tile of gemm_core.h, or, for d = 128 with an even head count, a 256-row
// tile of two heads with the two-group tile (the
// tiles of a row tile run on one XCD, one after the other, so the x tile is
// read from HBM once and from that XCD's L2 by the others). The epilogue rounds the tile to bf16 and passes it through LDS so that each
// lane writes 16 contiguous bytes of a row. For qk tiles the same pass produces
// what the hash's pre-pass would compute from these rows (the norm bounds of
// the rows' fp16 form and of its conversion error, and the squared norm),
// with the same per-row arithmetic, so the hash can skip that pass.
#include "dtype.h"
#include "gemm_core.h"
#include "hash_x16.h"
#include "internal.h"

namespace lsh {
namespace {

using gemm::floatx4_t;

using gemm::kThreads;
constexpr int kRows = 256;  // rows of x per tile
constexpr int kSlab = 32;   // K per LDS slab

template <int D>
struct PLds {
  static constexpr int kOutStride = D * 2 + 16;  // epilogue tile row (bf16, +pad)
  static constexpr int kMain = gemm::Lay<kRows, D, kSlab>::kBytes;
  static constexpr int kBytes = kMain > kRows * kOutStride ? kMain : kRows * kOutStride;
};

template <int D>
__global__ __launch_bounds__(kThreads, 2) void k_proj_mfma(
    const uint4* __restrict__ x, const uint4* __restrict__ w_qk, const uint4* __restrict__ w_v,
    uint4* __restrict__ qk, uint4* __restrict__ v,
    float2* __restrict__ xnorm, float* __restrict__ knorm, int64_t M, int L, int H,
    int model_dim) {
  using Lay = PLds<D>;
  extern __shared__ __align__(16) unsigned char lds[];
  // Workgroups are dealt to the 8 XCDs round-robin (XCD = blockIdx % 8): the
  // 2H tiles of a row tile get ids of one residue, consecutive within their
  // XCD, so the row tile of x is fetched into that XCD's L2 once.
  const unsigned nts = 2 * H;
  const unsigned xcd = blockIdx.x % 8u, k = blockIdx.x / 8u;
  const int nt = (int)(k % nts);
  const int64_t mt = (int64_t)(k / nts) * 8 + xcd;
  const int64_t row0 = mt * kRows;
  if (row0 >= M) return;
  const bool is_v = nt >= H;
  const int h = is_v ? nt - H : nt;
  const uint4* wrows = (is_v ? w_v : w_qk) + (int64_t)h * D * (model_dim / 8);
  const int t = threadIdx.x;

  constexpr int RT = gemm::Lay<kRows, D, kSlab>::RT, CT = gemm::Lay<kRows, D, kSlab>::CT;
  floatx4_t acc[RT][CT];
  gemm::tile<kRows, D, kSlab>(lds, x, row0, M, wrows, model_dim, acc);
  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const int wr = gemm::wave_row<kRows>(w), wc = gemm::wave_col<D>(w);

  // epilogue: lane holds rows wr + 16i + 4g + 0..3 of column wc + 16ct + lq;
  // the tile goes to LDS as bf16 rows, then out with 16 bytes per lane
  unsigned char* ot = lds;
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        *(uint16_t*)(ot + (wr + 16 * i + 4 * g + u) * Lay::kOutStride + (wc + 16 * ct + lq) * 2) =
            f32_to_bf16(acc[i][ct][u]).bits;
  __syncthreads();
  constexpr int kLpr = D / 8;                  // lanes per row (16 bytes each)
  constexpr int kRowsPerPass = kThreads / kLpr;
  const int sub = t % kLpr;
#pragma unroll
  for (int r0 = 0; r0 < kRows; r0 += kRowsPerPass) {
    const int r = r0 + t / kLpr;
    const int64_t row = row0 + r;  // a row of x: (b, i)
    const bool live = row < M;
    const int64_t b = row / L, i = row - b * L;
    const int64_t th = (b * H + h) * L + i;  // its token-head row
    const uint4 raw = *(const uint4*)(ot + r * Lay::kOutStride + sub * 16);
    if (live) (is_v ? v : qk)[th * kLpr + sub] = raw;
    if (!is_v) {  // the hash pre-pass of this row (all lanes of a row are live together)
      float bb = 0.f, c = 0.f;
      hx::x16_piece(raw, bb, c);
#pragma unroll
      for (int off = 1; off < kLpr; off <<= 1) {
        c += __shfl_xor(c, off);
        bb += __shfl_xor(bb, off);
      }
      if (live && sub == 0) {
        knorm[th] = c;
        xnorm[th] = hx::norm_bounds(c, bb);
      }
    }
  }
}

// d = 128 with an even head count: a 256-row x 256-column tile (heads 2p and
// 2p + 1 of qk or of v) on the two-group tile of gemm_core.h; its wave column
// w % 2 holds head 2p + w % 2.
// The epilogue takes one head at a time through LDS, with the same per-row
// arithmetic as k_proj_mfma.
constexpr int kPPOutStride = 128 * 2 + 16;
constexpr int kPPBytes =
    gemm::LayPP::kBytes > kRows * kPPOutStride ? gemm::LayPP::kBytes : kRows * kPPOutStride;

__global__ __launch_bounds__(gemm::LayPP::kThr, 1) void k_proj_pp(
    const uint4* __restrict__ x, const uint4* __restrict__ w_qk, const uint4* __restrict__ w_v,
    uint4* __restrict__ qk, uint4* __restrict__ v,
    float2* __restrict__ xnorm, float* __restrict__ knorm, int64_t M, int L, int H,
    int model_dim) {
  constexpr int D = 128;
  constexpr int kThr = gemm::LayPP::kThr;
  extern __shared__ __align__(16) unsigned char lds[];
  // the H tiles of a row tile (H/2 head pairs of qk, then of v) get ids of
  // one residue mod 8, consecutive within their XCD
  const unsigned nts = H;
  const unsigned xcd = blockIdx.x % 8u, k = blockIdx.x / 8u;
  const int nt = (int)(k % nts);
  const int64_t mt = (int64_t)(k / nts) * 8 + xcd;
  const int64_t row0 = mt * kRows;
  if (row0 >= M) return;
  const bool is_v = nt >= H / 2;
  const int h0 = 2 * (is_v ? nt - H / 2 : nt);
  const uint4* wrows = (is_v ? w_v : w_qk) + (int64_t)h0 * D * (model_dim / 8);
  const int t = threadIdx.x;

  floatx4_t acc[4][8];
  gemm::tile_pp(lds, x, row0, M, wrows, model_dim, acc);
  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const int wr = 64 * (w / 2), hh = w % 2;

  unsigned char* ot = lds;
  constexpr int kLpr = D / 8;  // lanes per row (16 bytes each)
  constexpr int kRowsPerPass = kThr / kLpr;
  const int sub = t % kLpr;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    // head h0 + pass: the waves of that column put it in LDS as bf16 rows
    if (hh == pass) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int u = 0; u < 4; ++u)
            *(uint16_t*)(ot + (wr + 16 * i + 4 * g + u) * kPPOutStride + (16 * ct + lq) * 2) =
                f32_to_bf16(acc[i][ct][u]).bits;
    }
    __syncthreads();
    const int h = h0 + pass;
#pragma unroll 2
    for (int r0 = 0; r0 < kRows; r0 += kRowsPerPass) {
      const int r = r0 + t / kLpr;
      const int64_t row = row0 + r;  // a row of x: (b, i)
      const bool live = row < M;
      const int64_t b = row / L, i = row - b * L;
      const int64_t th = (b * H + h) * L + i;  // its token-head row
      const uint4 raw = *(const uint4*)(ot + r * kPPOutStride + sub * 16);
      if (live) (is_v ? v : qk)[th * kLpr + sub] = raw;
      if (!is_v) {  // the hash pre-pass of this row (all lanes of a row are live together)
        float bb = 0.f, c = 0.f;
        hx::x16_piece(raw, bb, c);
#pragma unroll
        for (int off = 1; off < kLpr; off <<= 1) {
          c += __shfl_xor(c, off);
          bb += __shfl_xor(bb, off);
        }
        if (live && sub == 0) {
          knorm[th] = c;
          xnorm[th] = hx::norm_bounds(c, bb);
        }
      }
    }
    __syncthreads();
  }
}

// fp32 or other shapes: one thread per output element, fp32 sums in k order
template <typename T>
__global__ __launch_bounds__(256) void k_proj_simple(const T* __restrict__ x,
                                                     const T* __restrict__ w_qk,
                                                     const T* __restrict__ w_v,
                                                     T* __restrict__ qk, T* __restrict__ v,
                                                     int64_t n, int L, int H, int D,
                                                     int model_dim) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= 2 * n) return;
  const bool is_v = idx >= n;
  const int64_t o = is_v ? idx - n : idx;  // [B, H, L, D] element
  const int e = (int)(o % D);
  const int64_t th = o / D;
  const int64_t i = th % L, bh = th / L;
  const int hh = (int)(bh % H);
  const int64_t b = bh / H;
  const T* xr = x + (b * L + i) * model_dim;
  const T* wr = (is_v ? w_v : w_qk) + ((int64_t)hh * D + e) * model_dim;
  float s = 0.f;
  for (int k = 0; k < model_dim; ++k) s = fmaf(to_f32(xr[k]), to_f32(wr[k]), s);
  (is_v ? v : qk)[o] = from_f32<T>(s);
}

}  // namespace

bool project_mfma_supported(const Problem& p, int model_dim) {
  return p.dtype == LSH_ATTN_BF16 && (p.d == 64 || p.d == 128) && model_dim % kSlab == 0 &&
         model_dim <= (1 << 20) && hash_mfma_supported(p);
}

hipError_t launch_project(const Problem& p, int model_dim, const void* x, const void* w_qk,
                          const void* w_v, void* qk, void* v, HashScratch& hs, float* knorm,
                          bool* norms_ready, hipStream_t s) {
  const int64_t M = (int64_t)p.B * p.L;
  *norms_ready = false;
  if (project_mfma_supported(p, model_dim) && knorm) {
    // row tiles rounded up to a multiple of 8 (one per XCD); the extra
    // workgroups return at once
    const int64_t mts = (M + kRows - 1) / kRows;
    const unsigned grid = (unsigned)(((mts + 7) / 8) * 8 * 2 * p.H);
    if (p.d == 128 && p.H % 2 == 0) {
      const unsigned grid_pp = (unsigned)(((mts + 7) / 8) * 8 * p.H);
      if (!hs.proj_attr)
        (void)hipFuncSetAttribute((const void*)k_proj_pp,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, kPPBytes);
      hipLaunchKernelGGL(k_proj_pp, dim3(grid_pp), dim3(gemm::LayPP::kThr), kPPBytes, s,
                         (const uint4*)x, (const uint4*)w_qk, (const uint4*)w_v, (uint4*)qk,
                         (uint4*)v, (float2*)hs.xnorm, knorm, M, p.L, p.H, model_dim);
    } else if (p.d == 128) {
      constexpr int shmem = PLds<128>::kBytes;
      if (!hs.proj_attr)
        (void)hipFuncSetAttribute((const void*)k_proj_mfma<128>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
      hipLaunchKernelGGL(k_proj_mfma<128>, dim3(grid), dim3(kThreads), shmem, s,
                         (const uint4*)x, (const uint4*)w_qk, (const uint4*)w_v, (uint4*)qk,
                         (uint4*)v, (float2*)hs.xnorm, knorm, M, p.L, p.H,
                         model_dim);
    } else {
      constexpr int shmem = PLds<64>::kBytes;
      if (!hs.proj_attr)
        (void)hipFuncSetAttribute((const void*)k_proj_mfma<64>,
                                  hipFuncAttributeMaxDynamicSharedMemorySize, shmem);
      hipLaunchKernelGGL(k_proj_mfma<64>, dim3(grid), dim3(kThreads), shmem, s,
                         (const uint4*)x, (const uint4*)w_qk, (const uint4*)w_v, (uint4*)qk,
                         (uint4*)v, (float2*)hs.xnorm, knorm, M, p.L, p.H,
                         model_dim);
    }
    hs.proj_attr = true;
    *norms_ready = true;
    return hipGetLastError();
  }
  const int64_t n = p.n_token_heads() * p.d;
  const dim3 grid((unsigned)((2 * n + 255) / 256));
  if (p.dtype == LSH_ATTN_BF16)
    hipLaunchKernelGGL(k_proj_simple<bf16_t>, grid, dim3(256), 0, s, (const bf16_t*)x,
                       (const bf16_t*)w_qk, (const bf16_t*)w_v, (bf16_t*)qk, (bf16_t*)v, n, p.L,
                       p.H, p.d, model_dim);
  else
    hipLaunchKernelGGL(k_proj_simple<float>, grid, dim3(256), 0, s, (const float*)x,
                       (const float*)w_qk, (const float*)w_v, (float*)qk, (float*)v, n, p.L,
                       p.H, p.d, model_dim);
  return hipGetLastError();
}

}  // namespace lsh
