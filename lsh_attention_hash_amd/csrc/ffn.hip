// ffn.hip -- the chunked feed-forward half of the reversible block.
//
// Reformer overview (www.dtcms.com/a/488796.html), section 2.3: the
// reversible block computes y2 = x2 + FF(y1), and the feed-forward is applied
// to one chunk of rows at a time, the chunk outputs concatenated, so that only
// one chunk's hidden activations (d_ff per row, usually 4 d_model) exist at
// once. The Reformer summary (p2.ttnews.xyz), "FF layer chunking", splits the
// same half of the block. FF is taken as the plain two-layer feed-forward:
//   hidden = max(0, y1 W1^T + b1),   y2 = x2 + hidden W2^T + b2
// with W1 [d_ff, d_model] and W2 [d_model, d_ff] (linear-layer weights).
//
// Per chunk two launches: the first layer writes the chunk's hidden rows
// (bias and ReLU in the epilogue, rounded to the layer dtype) into the
// handle's buffer of chunk_rows x d_ff, and the second layer reads them back
// (bias and residual in its epilogue). Both use the tiles of gemm_core.h with
// K slabs of 32 on matrix cores for bf16 with d_model and d_ff multiples of
// 128: 256 x 256 tiles of 8 waves in two alternating groups (tile_pp, one
// workgroup per CU) for layers whose output width is a multiple of 256, else
// 256 x 128 tiles of 4 waves (two workgroups per CU);
// other shapes and fp32 use a plain kernel (one thread per output element).
// A row's result does not depend on the chunk it falls in: every output
// element is summed over K in the same order in any tile.
#include <vector>

#include "dtype.h"
#include "gemm_core.h"
#include "internal.h"
#include "lsh_attn.h"

namespace lsh {
namespace {

using gemm::floatx4_t;

constexpr int kBM = 256;       // rows per tile
constexpr int kKSlab = 32;     // K per LDS slab
constexpr int kGroupRows = 8;  // row tiles per group in an XCD's tile order

// Tile shape per output-column width BN: the wave grid (WM x WN waves) and
// the workgroups per CU the registers and LDS allow.
template <int BN>
struct FCfg;
template <>
struct FCfg<128> {
  static constexpr int WM = 2, WN = 2, kPerCU = 2;
};
template <>
struct FCfg<256> {
  static constexpr int WM = 4, WN = 2, kPerCU = 1;
};

template <int BN>
struct FLds {
  using C = FCfg<BN>;
  using Tile = gemm::Lay<kBM, BN, kKSlab, C::WM, C::WN>;
  static constexpr int kThr = Tile::kThr;
  static constexpr int kOutStride = BN * 4 + 16;  // epilogue slice row (fp32, +pad)
  static constexpr int kSlice = kBM / C::WM * kOutStride;  // one wave row's slice
  static constexpr int kTileBytes = BN == 256 ? gemm::LayPP::kBytes : Tile::kBytes;
  static constexpr int kBytes = kTileBytes > kSlice ? kTileBytes : kSlice;
};

// out[M, N] = epilogue(a[M, K] b[N, K]^T + bias[N]); UP: ReLU, else + resid
// (resid [M, N] or null). Row-major bf16, N a multiple of BN, K of 32.
template <bool UP, int BN>
__global__ __launch_bounds__(FLds<BN>::kThr, FCfg<BN>::kPerCU) void k_ffn_mfma(
    const uint4* __restrict__ a, const uint4* __restrict__ b, const bf16_t* __restrict__ bias,
    const uint4* resid, uint4* out, int64_t M, int N, int K,
    int mtl_n) {
  extern __shared__ __align__(16) unsigned char lds[];
  // Workgroups are dealt to the 8 XCDs round-robin (XCD = blockIdx % 8); XCD
  // x owns row tiles x, x + 8, ... Inside an XCD, tiles go in groups of
  // kGroupRows row tiles, row-fastest, so that the workgroups resident at
  // once share a few rows of a and a few column tiles of b in its L2.
  using C = FCfg<BN>;
  using Tile = typename FLds<BN>::Tile;
  constexpr int kThr = FLds<BN>::kThr;
  const int nts = N / BN;
  const int xcd = (int)(blockIdx.x % 8u);
  const int k = (int)(blockIdx.x / 8u);
  const int grp = k / (kGroupRows * nts);
  const int rem = k - grp * kGroupRows * nts;
  const int gm = min(kGroupRows, mtl_n - grp * kGroupRows);  // row tiles in this group
  const int64_t mt = (int64_t)(grp * kGroupRows + rem % gm) * 8 + xcd;
  const int nt = rem / gm;
  const int64_t row0 = mt * kBM;
  if (row0 >= M) return;
  const int n0 = nt * BN;

  constexpr int RT = Tile::RT, CT = Tile::CT;
  floatx4_t acc[RT][CT];
  if constexpr (BN == 256)
    gemm::tile_pp(lds, a, row0, M, b + (int64_t)n0 * (K / 8), K, acc);
  else
    gemm::tile<kBM, BN, kKSlab, C::WM, C::WN>(lds, a, row0, M, b + (int64_t)n0 * (K / 8), K, acc);
  const int t = threadIdx.x;
  const int lane = t & 63, w = t >> 6, g = lane >> 4, lq = lane & 15;
  const int wc = gemm::wave_col<BN, C::WN>(w);

  // epilogue in slices of kBM / WM rows (one row of waves at a time): bias
  // (and ReLU) on the lane's elements, the slice to LDS in fp32, then out by
  // rows, 8 elements (16 bytes of output) per lane
  float* ot = (float*)lds;
  constexpr int kOS = FLds<BN>::kOutStride / 4;
  float bv[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) bv[ct] = to_f32(bias[n0 + wc + 16 * ct + lq]);
  constexpr int kLpr = BN / 8;  // lanes per row
  constexpr int kRowsPerPass = kThr / kLpr;
  const int sub = t % kLpr;
  const int64_t ldo = N / 8;  // 16-byte pieces per output row
#pragma unroll
  for (int half = 0; half < C::WM; ++half) {
    if (w / C::WN == half) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int i = 0; i < RT; ++i)
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            float y = acc[i][ct][u] + bv[ct];
            if (UP) y = fmaxf(y, 0.f);
            ot[(16 * i + 4 * g + u) * kOS + wc + 16 * ct + lq] = y;
          }
    }
    __syncthreads();
#pragma unroll 2
    for (int r0 = 0; r0 < kBM / C::WM; r0 += kRowsPerPass) {
      const int r = r0 + t / kLpr;
      const int64_t row = row0 + half * (kBM / C::WM) + r;
      if (row >= M) continue;
      const float4 lo = *(const float4*)(ot + r * kOS + sub * 8);
      const float4 hi = *(const float4*)(ot + r * kOS + sub * 8 + 4);
      float y[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
      const int64_t off = row * ldo + n0 / 8 + sub;
      if (!UP && resid) {
        const uint4 rv = resid[off];
        const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          y[2 * q] += __uint_as_float(rw[q] << 16);
          y[2 * q + 1] += __uint_as_float(rw[q] & 0xFFFF0000u);
        }
      }
      uint32_t pw[4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
        pw[q] = (uint32_t)f32_to_bf16(y[2 * q]).bits |
                ((uint32_t)f32_to_bf16(y[2 * q + 1]).bits << 16);
      out[off] = uint4{pw[0], pw[1], pw[2], pw[3]};
    }
    __syncthreads();
  }
}

// Any shape, fp32 or bf16: one thread per output element, fp32 sums in K order.
template <typename T, bool UP>
__global__ __launch_bounds__(256) void k_ffn_simple(const T* __restrict__ a,
                                                    const T* __restrict__ b,
                                                    const T* __restrict__ bias,
                                                    const T* resid,
                                                    T* out, int64_t M, int N, int K) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= M * N) return;
  const int64_t m = idx / N;
  const int n = (int)(idx - m * N);
  const T* ar = a + m * K;
  const T* br = b + (int64_t)n * K;
  float s = 0.f;
  for (int k = 0; k < K; ++k) s = fmaf(to_f32(ar[k]), to_f32(br[k]), s);
  s += to_f32(bias[n]);
  if (UP) s = fmaxf(s, 0.f);
  if (!UP && resid) s += to_f32(resid[idx]);
  out[idx] = from_f32<T>(s);
}

bool ffn_mfma_supported(int dtype, int d_model, int d_ff) {
  return dtype == LSH_ATTN_BF16 && d_model % 128 == 0 && d_ff % 128 == 0 && d_model <= (1 << 20) &&
         d_ff <= (1 << 20);
}

template <bool UP, int BN>
void launch_mfma(const void* a, const void* b, const void* bias, const void* resid, void* out,
                 int64_t M, int N, int K, hipStream_t s) {
  const int64_t mts = (M + kBM - 1) / kBM;
  const int mtl_n = (int)((mts + 7) / 8);  // row tiles per XCD
  const unsigned grid = (unsigned)((int64_t)mtl_n * 8 * (N / BN));
  constexpr int shmem = FLds<BN>::kBytes;
  auto kern = k_ffn_mfma<UP, BN>;
  static bool configured[kMaxDevices] = {};
  if (first_on_device(configured)) {
    (void)hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              shmem);
  }
  hipLaunchKernelGGL(kern, dim3(grid), dim3(FLds<BN>::kThr), shmem, s, (const uint4*)a,
                     (const uint4*)b, (const bf16_t*)bias, (const uint4*)resid, (uint4*)out, M,
                     N, K, mtl_n);
}

// One layer over M rows: out = epilogue(a b^T + bias).
template <bool UP>
hipError_t launch_layer(int dtype, const void* a, const void* b, const void* bias,
                        const void* resid, void* out, int64_t M, int N, int K, bool mfma,
                        hipStream_t s) {
  if (mfma) {
    if (N % 256 == 0) launch_mfma<UP, 256>(a, b, bias, resid, out, M, N, K, s);
    else launch_mfma<UP, 128>(a, b, bias, resid, out, M, N, K, s);
  } else {
    const dim3 grid((unsigned)((M * N + 255) / 256));
    if (dtype == LSH_ATTN_BF16) {
      auto kern = k_ffn_simple<bf16_t, UP>;
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const bf16_t*)a, (const bf16_t*)b,
                         (const bf16_t*)bias, (const bf16_t*)resid, (bf16_t*)out, M, N, K);
    } else {
      auto kern = k_ffn_simple<float, UP>;
      hipLaunchKernelGGL(kern, grid, dim3(256), 0, s, (const float*)a, (const float*)b,
                         (const float*)bias, (const float*)resid, (float*)out, M, N, K);
    }
  }
  return hipGetLastError();
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

}  // namespace
}  // namespace lsh

struct lsh_ffn_s {
  int device = -1;
  lsh_ffn_config_t cfg{};
  int64_t chunk = 0;  // rows per chunk
  void* hidden = nullptr;
  int64_t bytes = 0;
  hipStream_t last_stream = nullptr;
  // timing: per timed forward, an event before the first launch and after each
  std::vector<hipEvent_t> events;
  std::vector<int> chunks;  // chunks of each timed forward
  int events_per_call = 0;
  int timing_capacity = 0, timed = 0;
};

namespace {

void ffn_destroy_events(lsh_ffn_s* h) {
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  h->events.clear();
  h->chunks.clear();
  h->timing_capacity = 0;
  h->timed = 0;
}

bool ffn_on_device(const lsh_ffn_s* h) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}

}  // namespace

extern "C" {

int lsh_ffn_create(const lsh_ffn_config_t* cfg, lsh_ffn_t* handle) {
  if (!handle) return LSH_ATTN_ERR_INVALID_ARG;
  *handle = nullptr;
  if (!cfg) return LSH_ATTN_ERR_INVALID_ARG;
  if (cfg->max_rows < 1 || cfg->d_model < 1 || cfg->d_ff < 1 || cfg->chunk_rows < 0)
    return LSH_ATTN_ERR_INVALID_ARG;
  if (cfg->dtype != LSH_ATTN_FP32 && cfg->dtype != LSH_ATTN_BF16) return LSH_ATTN_ERR_UNSUPPORTED;
  // 16-byte rows on the matrix-core path, and int32 columns everywhere
  if (cfg->d_model % 8 != 0 || cfg->d_ff % 8 != 0) return LSH_ATTN_ERR_UNSUPPORTED;
  const int64_t chunk = (cfg->chunk_rows == 0 || cfg->chunk_rows > cfg->max_rows)
                            ? cfg->max_rows
                            : cfg->chunk_rows;
  // the plain kernel's grid counts output elements of one chunk
  if (!lsh::ffn_mfma_supported(cfg->dtype, cfg->d_model, cfg->d_ff) &&
      chunk * (int64_t)(cfg->d_ff > cfg->d_model ? cfg->d_ff : cfg->d_model) > (1ll << 31))
    return LSH_ATTN_ERR_UNSUPPORTED;
  lsh_ffn_s* h = new lsh_ffn_s();
  h->cfg = *cfg;
  h->chunk = chunk;
  if (hipGetDevice(&h->device) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return LSH_ATTN_ERR_HIP;
  }
  const int64_t esize = cfg->dtype == LSH_ATTN_BF16 ? 2 : 4;
  h->bytes = h->chunk * cfg->d_ff * esize;
  if (hipMalloc(&h->hidden, (size_t)h->bytes) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return LSH_ATTN_ERR_OUT_OF_MEMORY;
  }
  const int64_t max_chunks = (cfg->max_rows + h->chunk - 1) / h->chunk;
  h->events_per_call = (int)(2 * max_chunks + 1);
  *handle = h;
  return LSH_ATTN_OK;
}

int lsh_ffn_forward(lsh_ffn_t h, int64_t rows, const void* y1, const void* w1, const void* b1,
                    const void* w2, const void* b2, const void* x2, void* y2, void* stream) {
  if (!h || rows < 0 || rows > h->cfg.max_rows) return LSH_ATTN_ERR_INVALID_ARG;
  if (!y1 || !w1 || !b1 || !w2 || !b2 || !y2) return LSH_ATTN_ERR_INVALID_ARG;
  if (!lsh::aligned16(y1) || !lsh::aligned16(w1) || !lsh::aligned16(w2) ||
      !lsh::aligned16(y2) || (x2 && !lsh::aligned16(x2)))
    return LSH_ATTN_ERR_INVALID_ARG;
  if (!ffn_on_device(h)) return LSH_ATTN_ERR_INVALID_ARG;
  if (rows == 0) return LSH_ATTN_OK;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  const lsh_ffn_config_t& c = h->cfg;
  const int64_t esize = c.dtype == LSH_ATTN_BF16 ? 2 : 4;
  const bool mfma = lsh::ffn_mfma_supported(c.dtype, c.d_model, c.d_ff);
  const int nch = (int)((rows + h->chunk - 1) / h->chunk);
  hipEvent_t* ev = nullptr;
  if (h->timed < h->timing_capacity) {
    ev = &h->events[(size_t)h->timed * h->events_per_call];
    h->chunks[h->timed] = nch;
    ++h->timed;
  }
  if (ev) (void)hipEventRecord(ev[0], s);
  hipError_t e = hipSuccess;
  for (int ci = 0; ci < nch && e == hipSuccess; ++ci) {
    const int64_t c0 = ci * h->chunk;
    const int64_t n = rows - c0 < h->chunk ? rows - c0 : h->chunk;
    const char* in = (const char*)y1 + c0 * c.d_model * esize;
    e = lsh::launch_layer<true>(c.dtype, in, w1, b1, nullptr, h->hidden, n, c.d_ff, c.d_model,
                                mfma, s);
    if (ev) (void)hipEventRecord(ev[2 * ci + 1], s);
    if (e != hipSuccess) break;
    const char* res = x2 ? (const char*)x2 + c0 * c.d_model * esize : nullptr;
    char* o = (char*)y2 + c0 * c.d_model * esize;
    e = lsh::launch_layer<false>(c.dtype, h->hidden, w2, b2, res, o, n, c.d_model, c.d_ff, mfma,
                                 s);
    if (ev) (void)hipEventRecord(ev[2 * ci + 2], s);
  }
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  return LSH_ATTN_OK;
}

int lsh_ffn_set_timing(lsh_ffn_t h, int capacity) {
  if (!h || capacity < 0) return LSH_ATTN_ERR_INVALID_ARG;
  if (!h->events.empty() && hipStreamSynchronize(h->last_stream) != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  ffn_destroy_events(h);
  const size_t n = (size_t)capacity * h->events_per_call;
  h->events.reserve(n);
  for (size_t k = 0; k < n; ++k) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      (void)hipGetLastError();
      ffn_destroy_events(h);
      return LSH_ATTN_ERR_HIP;
    }
    h->events.push_back(e);
  }
  h->chunks.assign((size_t)capacity, 0);
  h->timing_capacity = capacity;
  return LSH_ATTN_OK;
}

int lsh_ffn_get_timing(lsh_ffn_t h, double* ms, int64_t* n_forwards, int64_t* n_chunks) {
  if (!h || !ms || !n_forwards || h->timing_capacity == 0) return LSH_ATTN_ERR_INVALID_ARG;
  ms[0] = ms[1] = 0.0;
  int64_t total = 0;
  for (int k = 0; k < h->timed; ++k) {
    const hipEvent_t* ev = &h->events[(size_t)k * h->events_per_call];
    const int nch = h->chunks[k];
    if (hipEventSynchronize(ev[2 * nch]) != hipSuccess) {
      (void)hipGetLastError();
      return LSH_ATTN_ERR_HIP;
    }
    for (int j = 0; j < 2 * nch; ++j) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, ev[j], ev[j + 1]) != hipSuccess) {
        (void)hipGetLastError();
        return LSH_ATTN_ERR_HIP;
      }
      ms[j % 2] += t;
    }
    total += nch;
  }
  *n_forwards = h->timed;
  if (n_chunks) *n_chunks = total;
  h->timed = 0;
  return LSH_ATTN_OK;
}

int lsh_ffn_workspace_bytes(lsh_ffn_t h, int64_t* bytes) {
  if (!h || !bytes) return LSH_ATTN_ERR_INVALID_ARG;
  *bytes = h->bytes;
  return LSH_ATTN_OK;
}

int lsh_ffn_destroy(lsh_ffn_t h) {
  if (!h) return LSH_ATTN_OK;
  int prev = -1;
  const bool switched = hipGetDevice(&prev) == hipSuccess && prev != h->device &&
                        hipSetDevice(h->device) == hipSuccess;
  const hipError_t e = hipDeviceSynchronize();
  ffn_destroy_events(h);
  (void)hipFree(h->hidden);
  if (switched) (void)hipSetDevice(prev);
  delete h;
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  return LSH_ATTN_OK;
}

}  // extern "C"
