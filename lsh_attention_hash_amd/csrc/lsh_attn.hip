// lsh_attn.hip -- host side of the C ABI declared in include/lsh_attn.h:
// argument checks, the workspace, and the launch sequence
//   hash -> sort -> (gather) -> chunked attention -> combine
// on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "internal.h"
#include "lsh_attn.h"

struct lsh_attn_s {
  lsh::Problem p;
  lsh::Workspace ws;
  lsh::BwdWorkspace bw;
  int device = 0;
  int64_t bytes = 0;
  hipStream_t last_stream = nullptr;
  // stage timing: events[k * kEvPerCall + j] marks the start of stage j of
  // timed forward k for j < 7 (j = 7: the end of stage 6); j = 8, 9 bracket
  // the projection (stage 7) of a forward from x, projected[k] says whether
  // it ran
  std::vector<hipEvent_t> events;
  std::vector<char> projected;
  int timing_capacity = 0;
  int timed = 0;
  // the same for backwards: bevents[k * (N_BWD_STAGES + 1) + j]
  std::vector<hipEvent_t> bevents;
  int btimed = 0;
};

namespace {

constexpr int kEvPerCall = LSH_ATTN_N_STAGES + 2;

__global__ void k_zero_u64(unsigned long long* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0ull;
}

lsh::Problem problem_of(const lsh_attn_config_t* c) {
  return lsh::Problem{c->batch,     c->heads,    c->seq_len,   c->head_dim,
                      c->n_buckets, c->n_rounds, c->chunk_len, c->causal,
                      c->dtype,     c->out_dtype, c->flags};
}

int validate(const lsh_attn_config_t* c) {
  if (!c) return LSH_ATTN_ERR_INVALID_ARG;
  if (c->batch < 1 || c->heads < 1 || c->seq_len < 1 || c->head_dim < 1)
    return LSH_ATTN_ERR_INVALID_ARG;
  if (c->seq_len > (1 << 24)) return LSH_ATTN_ERR_INVALID_ARG;
  if (c->n_rounds < 1 || c->chunk_len < 1 || c->seq_len % c->chunk_len != 0)
    return LSH_ATTN_ERR_INVALID_ARG;
  if (c->n_buckets < 1 || c->n_buckets > 65536 || (c->n_buckets > 1 && c->n_buckets % 2 != 0))
    return LSH_ATTN_ERR_INVALID_ARG;
  if (c->causal != 0 && c->causal != 1) return LSH_ATTN_ERR_INVALID_ARG;
  if ((c->flags & ~(LSH_ATTN_FLAG_SEPARATE_GATHER | LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS |
                    LSH_ATTN_FLAG_BACKWARD | lsh::kVariantFlags)) != 0)
    return LSH_ATTN_ERR_INVALID_ARG;
  if (c->dtype != LSH_ATTN_FP32 && c->dtype != LSH_ATTN_BF16) return LSH_ATTN_ERR_UNSUPPORTED;
  if (c->out_dtype != LSH_ATTN_FP32 && c->out_dtype != LSH_ATTN_BF16)
    return LSH_ATTN_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return LSH_ATTN_ERR_UNSUPPORTED;
  if (c->chunk_len > 256) return LSH_ATTN_ERR_UNSUPPORTED;
  return LSH_ATTN_OK;
}

void free_ws(lsh::Workspace& w) {
  (void)hipFree(w.buckets);
  (void)hipFree(w.perm);
  (void)hipFree(w.inv);
  (void)hipFree(w.o);
  (void)hipFree(w.lse);
  (void)hipFree(w.sort_counts);
  (void)hipFree(w.qk_sorted);
  (void)hipFree(w.v_sorted);
  (void)hipFree(w.stats);
  (void)hipFree(w.knorm);
  (void)hipFree(w.hash.rh);
  (void)hipFree(w.hash.rt);
  (void)hipFree(w.hash.bounds);
  (void)hipFree(w.hash.queue_a);
  (void)hipFree(w.hash.queue_b);
  (void)hipFree(w.hash.xnorm);
  w = lsh::Workspace{};
}

void free_bw(lsh::BwdWorkspace& b) {
  (void)hipFree(b.o32);
  (void)hipFree(b.od);
  (void)hipFree(b.lse);
  (void)hipFree(b.w);
  (void)hipFree(b.cq);
  (void)hipFree(b.wself);
  (void)hipFree(b.dq);
  (void)hipFree(b.dk);
  (void)hipFree(b.dv);
  b = lsh::BwdWorkspace{};
}

template <typename T>
bool alloc(T** ptr, int64_t bytes, int64_t& total) {
  void* q = nullptr;
  if (hipMalloc(&q, (size_t)(bytes > 0 ? bytes : 1)) != hipSuccess) {
    (void)hipGetLastError();  // clear the sticky error of the failed allocation
    return false;
  }
  *ptr = (T*)q;
  total += bytes;
  return true;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// The forward's workspace buffers for a problem, in one order: where each
// pointer goes and how many bytes it takes. create allocates each one; the
// allocation-free forward carves them out of its static scratch.
struct Part {
  void** ptr;
  int64_t bytes;
};
constexpr int kMaxParts = 20;
int forward_parts(const lsh::Problem& p, lsh::Workspace& w, Part* parts) {
  const int64_t rows = p.n_rows();
  const int esize = p.dtype == LSH_ATTN_BF16 ? 2 : 4;
  int n = 0;
  auto add = [&](auto** ptr, int64_t bytes) { parts[n++] = Part{(void**)ptr, bytes}; };
  add(&w.buckets, rows * 2);
  add(&w.perm, rows * 4);
  add(&w.o, p.nseg() * p.o_seg_rows() * p.d * (lsh::round_outputs_half(p) ? 2 : 4));
  add(&w.lse, rows * 4);
  add(&w.sort_counts, p.nseg() * (int64_t)p.nb * (p.sort_tiles() + 2) * 4);
  add(&w.stats, 4 * 8);
  if (lsh::attend_mfma_supported(p) || lsh::attend_variant_mfma_supported(p))
    add(&w.knorm, p.n_token_heads() * 4);
  if (lsh::hash_mfma_supported(p)) {
    const int64_t hp = lsh::hash_half_pad(p);
    add(&w.hash.rh, (int64_t)p.R * hp * p.d * 2);
    add(&w.hash.rt, (int64_t)p.R * p.half() * p.d * 4);
    add(&w.hash.bounds, (4 * (int64_t)p.R * (hp / 32) + 2) * 4);
    add(&w.hash.queue_a, rows * 16);
    add(&w.hash.queue_b, rows * 8);
    add(&w.hash.xnorm, p.n_token_heads() * 8);
  }
  if (p.flags & LSH_ATTN_FLAG_DEDUP) add(&w.inv, rows * 4);
  if (p.flags & LSH_ATTN_FLAG_SEPARATE_GATHER) {
    add(&w.qk_sorted, rows * p.d * esize);
    add(&w.v_sorted, rows * p.d * esize);
  }
  return n;
}

// compute units of the current device (1 if the query fails)
int device_cus(int device) {
  int n_cu = 1;
  if (hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, device) !=
          hipSuccess ||
      n_cu < 1) {
    (void)hipGetLastError();
    n_cu = 1;
  }
  return n_cu;
}

}  // namespace

extern "C" {

int lsh_attn_create(const lsh_attn_config_t* cfg, lsh_attn_t* handle) {
  if (!handle) return LSH_ATTN_ERR_INVALID_ARG;
  *handle = nullptr;
  const int rc = validate(cfg);
  if (rc != LSH_ATTN_OK) return rc;
  lsh_attn_s* h = new (std::nothrow) lsh_attn_s();
  if (!h) return LSH_ATTN_ERR_OUT_OF_MEMORY;
  h->p = problem_of(cfg);
  if (hipGetDevice(&h->device) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return LSH_ATTN_ERR_HIP;
  }
  const lsh::Problem& p = h->p;
  const int64_t rows = p.n_rows();
  lsh::Workspace& w = h->ws;
  int64_t& t = h->bytes;
  Part parts[kMaxParts];
  const int np = forward_parts(p, w, parts);
  bool ok = true;
  for (int i = 0; ok && i < np; ++i) ok = alloc(parts[i].ptr, parts[i].bytes, t);
  ok = ok && hipMemset(w.stats, 0, 4 * 8) == hipSuccess;
  if (ok && lsh::hash_mfma_supported(p)) w.hash.n_cu = device_cus(h->device);
  if (ok && (p.flags & LSH_ATTN_FLAG_BACKWARD)) {
    lsh::BwdWorkspace& b = h->bw;
    ok = (lsh::bwd_recompute_dot(p) ? alloc(&b.od, rows * 4, t)
                                    : alloc(&b.o32, p.nseg() * p.o_seg_rows() * p.d * 4, t)) &&
         alloc(&b.lse, rows * 4, t) &&
         alloc(&b.w, rows * 4, t) && alloc(&b.cq, p.n_token_heads() * 4, t) &&
         alloc(&b.wself, p.n_token_heads() * 4, t) &&
         alloc(&b.dq, rows * p.d * (lsh::bwd_rows_half(p) ? 2 : 4), t) &&
         (lsh::bwd_mfma_supported(p) || alloc(&b.dk, rows * p.d * 4, t)) &&
         alloc(&b.dv, rows * p.d * (lsh::bwd_rows_half(p) ? 2 : 4), t);
  }
  if (!ok) {
    free_bw(h->bw);
    free_ws(w);
    delete h;
    return LSH_ATTN_ERR_OUT_OF_MEMORY;
  }
  *handle = h;
  return LSH_ATTN_OK;
}

namespace {

// The forward after the inputs are checked; ev: the timed call's events or
// null; norms_ready: the projection already wrote the hash's row norm bounds.
int forward_body(const lsh::Problem& p, lsh::Workspace& w, const void* qk, const void* v,
                 const float* rotations, void* out, float* lse, int32_t* buckets, int32_t* perm,
                 hipStream_t s, hipEvent_t* ev, bool norms_ready) {
  auto mark = [&](int j) {
    if (ev) (void)hipEventRecord(ev[j], s);
  };
  int32_t* pm = perm ? perm : w.perm;
  float* ls = lse ? lse : w.lse;
  hipError_t e = hipSuccess;
  const bool mfma_hash = lsh::hash_mfma_supported(p);
  // the matrix-core hash reports its own re-scoring counts
  if (!mfma_hash) hipLaunchKernelGGL(k_zero_u64, dim3(1), dim3(64), 0, s, w.stats, 2);
  mark(0);
  if (e == hipSuccess) {
    if (mfma_hash) {
      e = lsh::launch_hash_mfma(p, qk, rotations, w.hash, w.buckets, buckets, w.stats, w.knorm, s,
                                ev ? ev[1] : nullptr, ev ? ev[2] : nullptr, norms_ready);
    } else {
      if (w.knorm) e = lsh::launch_key_norms(p, qk, w.knorm, s);
      mark(1);
      if (e == hipSuccess) e = lsh::launch_hash_exact(p, qk, rotations, w.buckets, buckets, s);
      mark(2);
    }
  }
  mark(3);
  if (e == hipSuccess) e = lsh::launch_sort(p, w.buckets, w.sort_counts, pm, s);
  mark(4);
  const bool separate = (p.flags & LSH_ATTN_FLAG_SEPARATE_GATHER) != 0;
  if (e == hipSuccess && separate)
    e = lsh::launch_gather(p, qk, v, pm, w.qk_sorted, w.v_sorted, s);
  mark(5);
  if (e == hipSuccess && (p.flags & LSH_ATTN_FLAG_DEDUP)) e = lsh::launch_inverse_perm(p, pm, w.inv, s);
  if (e == hipSuccess)
    e = lsh::launch_attend(p, qk, v, separate ? w.qk_sorted : nullptr,
                           separate ? w.v_sorted : nullptr, pm, w.knorm, w.buckets, w.inv,
                           (float*)w.o, ls, s);
  mark(6);
  if (e == hipSuccess)
    e = lsh::launch_combine(p, w.o, lsh::round_outputs_half(p), ls, v, out, w.stats + 2, s);
  mark(7);
  if (e == hipSuccess) e = hipGetLastError();
  return e == hipSuccess ? LSH_ATTN_OK : LSH_ATTN_ERR_HIP;
}

// the next timed call's events (null when not timing)
hipEvent_t* next_events(lsh_attn_s* h, bool projected) {
  if (h->timed >= h->timing_capacity) return nullptr;
  hipEvent_t* ev = &h->events[(size_t)h->timed * kEvPerCall];
  h->projected[h->timed] = projected ? 1 : 0;
  ++h->timed;
  return ev;
}

// A call that failed before recording all of its events gives its timing slot
// back, so the accumulation only holds calls whose events were all recorded.
int release_on_error(lsh_attn_s* h, const hipEvent_t* ev, int rc) {
  if (rc != LSH_ATTN_OK && ev && h->timed > 0) --h->timed;
  return rc;
}

bool on_device(const lsh_attn_s* h) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev != h->device) {
    (void)hipGetLastError();
    return false;
  }
  return true;
}

}  // namespace

int lsh_attn_forward(lsh_attn_t h, const void* qk, const void* v, const float* rotations,
                     void* out, float* lse, int32_t* buckets, int32_t* perm, void* stream) {
  if (!h || !qk || !v || !out) return LSH_ATTN_ERR_INVALID_ARG;
  if (h->p.nb > 1 && !rotations) return LSH_ATTN_ERR_INVALID_ARG;
  if (!aligned16(qk) || !aligned16(v) || !aligned16(out)) return LSH_ATTN_ERR_INVALID_ARG;
  if (!on_device(h)) return LSH_ATTN_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  hipEvent_t* ev = next_events(h, false);
  return release_on_error(h, ev,
                          forward_body(h->p, h->ws, qk, v, rotations, out, lse, buckets, perm, s,
                                       ev, false));
}

int lsh_attn_forward_x(lsh_attn_t h, const void* x, int32_t model_dim, const void* w_qk,
                       const void* w_v, const float* rotations, void* qk, void* v, void* out,
                       float* lse, int32_t* buckets, int32_t* perm, void* stream) {
  if (!h || !x || !w_qk || !w_v || !qk || !v || !out) return LSH_ATTN_ERR_INVALID_ARG;
  if (model_dim < 1 || (int64_t)model_dim * h->p.d * h->p.H > ((int64_t)1 << 31))
    return LSH_ATTN_ERR_INVALID_ARG;
  if (h->p.nb > 1 && !rotations) return LSH_ATTN_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_qk) || !aligned16(w_v) || !aligned16(qk) || !aligned16(v) ||
      !aligned16(out))
    return LSH_ATTN_ERR_INVALID_ARG;
  if (!on_device(h)) return LSH_ATTN_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  hipEvent_t* ev = next_events(h, true);
  if (ev) (void)hipEventRecord(ev[8], s);
  bool norms_ready = false;
  const hipError_t e = lsh::launch_project(h->p, model_dim, x, w_qk, w_v, qk, v, h->ws.hash,
                                           h->ws.knorm, &norms_ready, s);
  if (ev) (void)hipEventRecord(ev[9], s);
  if (e != hipSuccess) return release_on_error(h, ev, LSH_ATTN_ERR_HIP);
  return release_on_error(
      h, ev,
      forward_body(h->p, h->ws, qk, v, rotations, out, lse, buckets, perm, s, ev, norms_ready));
}

int lsh_attn_backward_buckets(lsh_attn_t h, const void* qk, const void* v, const int32_t* perm,
                              const int32_t* buckets, const void* dout, void* dqk, void* dv,
                              void* stream) {
  if (!h || !qk || !v || !perm || !dout || !dqk || !dv) return LSH_ATTN_ERR_INVALID_ARG;
  const lsh::Problem& p = h->p;
  if (!(p.flags & LSH_ATTN_FLAG_BACKWARD)) return LSH_ATTN_ERR_UNSUPPORTED;
  if ((p.flags & LSH_ATTN_FLAG_SAME_BUCKET) && !buckets) return LSH_ATTN_ERR_INVALID_ARG;
  if (!aligned16(qk) || !aligned16(v) || !aligned16(dout) || !aligned16(dqk) || !aligned16(dv))
    return LSH_ATTN_ERR_INVALID_ARG;
  if (!on_device(h)) return LSH_ATTN_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  const bool timing = h->btimed < h->timing_capacity;
  const hipEvent_t* ev =
      timing ? &h->bevents[(size_t)h->btimed * (LSH_ATTN_N_BWD_STAGES + 1)] : nullptr;
  if (timing) ++h->btimed;
  hipError_t e = lsh::launch_backward(p, qk, v, perm, buckets, dout, dqk, dv, h->ws.knorm,
                                      h->ws.buckets, h->ws.inv, h->bw, h->ws.stats + 3, s, ev);
  if (e == hipSuccess) e = hipGetLastError();
  if (e != hipSuccess && timing) --h->btimed;  // its events were not all recorded
  return e == hipSuccess ? LSH_ATTN_OK : LSH_ATTN_ERR_HIP;
}

int lsh_attn_backward(lsh_attn_t h, const void* qk, const void* v, const int32_t* perm,
                      const void* dout, void* dqk, void* dv, void* stream) {
  return lsh_attn_backward_buckets(h, qk, v, perm, nullptr, dout, dqk, dv, stream);
}

int lsh_attn_get_stats(lsh_attn_t h, lsh_attn_stats_t* stats) {
  if (!h || !stats) return LSH_ATTN_ERR_INVALID_ARG;
  unsigned long long host[4] = {0, 0, 0, 0};
  const unsigned long long zero[2] = {0, 0};
  if (hipStreamSynchronize(h->last_stream) != hipSuccess ||
      hipMemcpy(host, h->ws.stats, sizeof(host), hipMemcpyDeviceToHost) != hipSuccess ||
      hipMemcpy(h->ws.stats + 2, zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  stats->n_exact_rescored = (int64_t)host[0];
  stats->n_full_fallback = (int64_t)host[1];
  stats->n_round_rows_at_fp16_limit = (int64_t)host[2];
  stats->n_grad_rows_at_fp16_limit = (int64_t)host[3];
  return LSH_ATTN_OK;
}

static void destroy_events(lsh_attn_s* h) {
  for (hipEvent_t e : h->events) (void)hipEventDestroy(e);
  for (hipEvent_t e : h->bevents) (void)hipEventDestroy(e);
  h->events.clear();
  h->bevents.clear();
  h->projected.clear();
  h->timing_capacity = 0;
  h->timed = 0;
  h->btimed = 0;
}

// capacity * per events into v (false if one cannot be created)
static bool create_events(std::vector<hipEvent_t>& v, size_t n) {
  v.reserve(n);
  for (size_t k = 0; k < n; ++k) {
    hipEvent_t e;
    if (hipEventCreate(&e) != hipSuccess) {
      (void)hipGetLastError();
      return false;
    }
    v.push_back(e);
  }
  return true;
}

// Sum over the first `count` timed calls of each of `stages` stage durations.
static int sum_stage_times(const std::vector<hipEvent_t>& events, int count, int stages,
                           double* ms) {
  for (int j = 0; j < stages; ++j) ms[j] = 0.0;
  for (int k = 0; k < count; ++k) {
    const hipEvent_t* ev = &events[(size_t)k * (stages + 1)];
    if (hipEventSynchronize(ev[stages]) != hipSuccess) {
      (void)hipGetLastError();
      return LSH_ATTN_ERR_HIP;
    }
    for (int j = 0; j < stages; ++j) {
      float t = 0.f;
      if (hipEventElapsedTime(&t, ev[j], ev[j + 1]) != hipSuccess) {
        (void)hipGetLastError();
        return LSH_ATTN_ERR_HIP;
      }
      ms[j] += t;
    }
  }
  return LSH_ATTN_OK;
}

int lsh_attn_set_timing(lsh_attn_t h, int capacity) {
  if (!h || capacity < 0) return LSH_ATTN_ERR_INVALID_ARG;
  if (!h->events.empty() && hipStreamSynchronize(h->last_stream) != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  destroy_events(h);
  h->projected.assign((size_t)capacity, 0);
  if (!create_events(h->events, (size_t)capacity * kEvPerCall) ||
      ((h->p.flags & LSH_ATTN_FLAG_BACKWARD) &&
       !create_events(h->bevents, (size_t)capacity * (LSH_ATTN_N_BWD_STAGES + 1)))) {
    destroy_events(h);
    return LSH_ATTN_ERR_HIP;
  }
  h->timing_capacity = capacity;
  return LSH_ATTN_OK;
}

int lsh_attn_get_timing(lsh_attn_t h, double* ms, int64_t* n_forwards) {
  if (!h || !ms || !n_forwards || h->timing_capacity == 0) return LSH_ATTN_ERR_INVALID_ARG;
  for (int j = 0; j < LSH_ATTN_N_STAGES; ++j) ms[j] = 0.0;
  for (int k = 0; k < h->timed; ++k) {
    const hipEvent_t* ev = &h->events[(size_t)k * kEvPerCall];
    if (hipEventSynchronize(ev[7]) != hipSuccess) {
      (void)hipGetLastError();
      return LSH_ATTN_ERR_HIP;
    }
    for (int j = 0; j < 8; ++j) {
      if (j == 7 && !h->projected[k]) break;
      float t = 0.f;
      const hipError_t e = j < 7 ? hipEventElapsedTime(&t, ev[j], ev[j + 1])
                                 : hipEventElapsedTime(&t, ev[8], ev[9]);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        return LSH_ATTN_ERR_HIP;
      }
      ms[j] += t;
    }
  }
  *n_forwards = h->timed;
  h->timed = 0;
  return LSH_ATTN_OK;
}

int lsh_attn_get_backward_timing(lsh_attn_t h, double* ms, int64_t* n_backwards) {
  if (!h || !ms || !n_backwards || h->timing_capacity == 0) return LSH_ATTN_ERR_INVALID_ARG;
  const int rc = sum_stage_times(h->bevents, h->btimed, LSH_ATTN_N_BWD_STAGES, ms);
  if (rc != LSH_ATTN_OK) return rc;
  *n_backwards = h->btimed;
  h->btimed = 0;
  return LSH_ATTN_OK;
}

int lsh_attn_workspace_bytes(lsh_attn_t h, int64_t* bytes) {
  if (!h || !bytes) return LSH_ATTN_ERR_INVALID_ARG;
  *bytes = h->bytes;
  return LSH_ATTN_OK;
}

int lsh_attn_destroy(lsh_attn_t h) {
  if (!h) return LSH_ATTN_OK;
  int prev = -1;
  const bool switched = hipGetDevice(&prev) == hipSuccess && prev != h->device &&
                        hipSetDevice(h->device) == hipSuccess;
  const hipError_t e = hipDeviceSynchronize();
  destroy_events(h);
  free_bw(h->bw);
  free_ws(h->ws);
  if (switched) (void)hipSetDevice(prev);
  delete h;
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  return LSH_ATTN_OK;
}

}  // extern "C"

// ---------------------------------------------------------------------------
// The allocation-free forward. Its workspace is carved from `scratch`, a
// static device array of kStaticScratchBytes that every GPU the library runs
// on holds for the life of the process. In host code the array's name is only
// a stand-in: its device address comes from hipGetSymbolAddress, once per
// device (with that device current), and only that address is used.
namespace {

constexpr int64_t kStaticScratchBytes = (int64_t)64 << 20;  // LSH_ATTN_STATIC_SCRATCH_BYTES
static_assert(kStaticScratchBytes == LSH_ATTN_STATIC_SCRATCH_BYTES, "header and source agree");
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
struct StaticDevice {
  void* ptr = nullptr;  // device address of this device's scratch
  int n_cu = 0;
  int hash_per_cu = 0;  // the hash kernel's resident workgroups per CU (0: not yet queried)
  bool proj_attr = false;
};
StaticDevice g_static[kMaxDevices];
std::mutex g_static_mutex;

// Set-up on the current device (first call there): the scratch's address.
int static_device(int device, StaticDevice** out) {
  if (device < 0 || device >= kMaxDevices) return LSH_ATTN_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_static_mutex);
  StaticDevice& sd = g_static[device];
  if (!sd.ptr) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return LSH_ATTN_ERR_HIP;
    }
    sd.n_cu = device_cus(device);
    sd.ptr = ptr;
  }
  *out = &sd;
  return LSH_ATTN_OK;
}

// bytes of the forward's workspace parts, each rounded up to 256
int64_t static_bytes(const lsh::Problem& p) {
  lsh::Workspace w;
  Part parts[kMaxParts];
  const int np = forward_parts(p, w, parts);
  int64_t total = 0;
  for (int i = 0; i < np; ++i) total += (parts[i].bytes + 255) / 256 * 256;
  return total;
}

}  // namespace

extern "C" {

int lsh_attn_forward_static(const lsh_attn_config_t* cfg, const void* qk, const void* v,
                            const float* rotations, void* out, float* lse, int32_t* buckets,
                            int32_t* perm, void* stream) {
  int rc = validate(cfg);
  if (rc != LSH_ATTN_OK) return rc;
  if (cfg->flags & LSH_ATTN_FLAG_BACKWARD) return LSH_ATTN_ERR_UNSUPPORTED;
  if (!qk || !v || !out) return LSH_ATTN_ERR_INVALID_ARG;
  if (cfg->n_buckets > 1 && !rotations) return LSH_ATTN_ERR_INVALID_ARG;
  if (!aligned16(qk) || !aligned16(v) || !aligned16(out)) return LSH_ATTN_ERR_INVALID_ARG;
  const lsh::Problem p = problem_of(cfg);
  if (static_bytes(p) > kStaticScratchBytes) return LSH_ATTN_ERR_WORKSPACE_TOO_LARGE;
  int device = -1;
  if (hipGetDevice(&device) != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  StaticDevice* sd = nullptr;
  rc = static_device(device, &sd);
  if (rc != LSH_ATTN_OK) return rc;
  lsh::Workspace w;
  Part parts[kMaxParts];
  const int np = forward_parts(p, w, parts);
  unsigned char* base = (unsigned char*)sd->ptr;
  int64_t off = 0;
  for (int i = 0; i < np; ++i) {
    *parts[i].ptr = base + off;
    off += (parts[i].bytes + 255) / 256 * 256;
  }
  w.hash.n_cu = sd->n_cu;
  w.hash.per_cu = sd->hash_per_cu;
  w.hash.proj_attr = sd->proj_attr;
  hipStream_t s = (hipStream_t)stream;
  rc = forward_body(p, w, qk, v, rotations, out, lse, buckets, perm, s, nullptr, false);
  sd->hash_per_cu = w.hash.per_cu;
  return rc;
}

const char* lsh_attn_strerror(int status) {
  switch (status) {
    case LSH_ATTN_OK: return "ok";
    case LSH_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case LSH_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case LSH_ATTN_ERR_OUT_OF_MEMORY: return "out of device memory";
    case LSH_ATTN_ERR_HIP: return "HIP runtime or launch error";
    case LSH_ATTN_ERR_WORKSPACE_TOO_LARGE:
      return "workspace larger than the static scratch of lsh_attn_forward_static (64 MiB)";
    default: return "unknown status";
  }
}

}  // extern "C"
