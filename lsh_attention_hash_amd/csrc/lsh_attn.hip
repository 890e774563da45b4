// lsh_attn.hip -- host side of the C ABI declared in include/lsh_attn.h:
// argument checks, the workspace, and the launch sequence
//   hash -> sort -> (gather) -> chunked attention -> combine
// on the caller's stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

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
  if ((c->flags & LSH_ATTN_FLAG_BACKWARD) && (c->flags & lsh::kVariantFlags))
    return LSH_ATTN_ERR_UNSUPPORTED;
  if (c->dtype != LSH_ATTN_FP32 && c->dtype != LSH_ATTN_BF16) return LSH_ATTN_ERR_UNSUPPORTED;
  if (c->out_dtype != LSH_ATTN_FP32 && c->out_dtype != LSH_ATTN_BF16)
    return LSH_ATTN_ERR_UNSUPPORTED;
  if (c->head_dim != 64 && c->head_dim != 128) return LSH_ATTN_ERR_UNSUPPORTED;
  if (c->chunk_len > 256) return LSH_ATTN_ERR_UNSUPPORTED;
  return LSH_ATTN_OK;
}

void free_ws(lsh::Workspace& w) {
  hipFree(w.buckets);
  hipFree(w.perm);
  hipFree(w.inv);
  hipFree(w.o);
  hipFree(w.lse);
  hipFree(w.sort_counts);
  hipFree(w.qk_sorted);
  hipFree(w.v_sorted);
  hipFree(w.stats);
  hipFree(w.knorm);
  hipFree(w.hash.rh);
  hipFree(w.hash.rt);
  hipFree(w.hash.bounds);
  hipFree(w.hash.queue_a);
  hipFree(w.hash.queue_b);
  hipFree(w.hash.x16);
  hipFree(w.hash.xnorm);
  w = lsh::Workspace{};
}

void free_bw(lsh::BwdWorkspace& b) {
  hipFree(b.o32);
  hipFree(b.od);
  hipFree(b.lse);
  hipFree(b.w);
  hipFree(b.cq);
  hipFree(b.wself);
  hipFree(b.dq);
  hipFree(b.dk);
  hipFree(b.dv);
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

}  // namespace

extern "C" {

int lsh_attn_create(const lsh_attn_config_t* cfg, lsh_attn_t* handle) {
  if (!handle) return LSH_ATTN_ERR_INVALID_ARG;
  *handle = nullptr;
  const int rc = validate(cfg);
  if (rc != LSH_ATTN_OK) return rc;
  lsh_attn_s* h = new (std::nothrow) lsh_attn_s();
  if (!h) return LSH_ATTN_ERR_OUT_OF_MEMORY;
  h->p = lsh::Problem{cfg->batch,  cfg->heads,   cfg->seq_len, cfg->head_dim,
                      cfg->n_buckets, cfg->n_rounds, cfg->chunk_len, cfg->causal,
                      cfg->dtype,  cfg->out_dtype, cfg->flags};
  if (hipGetDevice(&h->device) != hipSuccess) {
    (void)hipGetLastError();
    delete h;
    return LSH_ATTN_ERR_HIP;
  }
  const lsh::Problem& p = h->p;
  const int64_t rows = p.n_rows();
  const int esize = p.dtype == LSH_ATTN_BF16 ? 2 : 4;
  lsh::Workspace& w = h->ws;
  int64_t& t = h->bytes;
  bool ok = alloc(&w.buckets, rows * 2, t) && alloc(&w.perm, rows * 4, t) &&
            alloc(&w.o, p.nseg() * p.o_seg_rows() * p.d * (lsh::round_outputs_half(p) ? 2 : 4), t) &&
            alloc(&w.lse, rows * 4, t) &&
            alloc(&w.sort_counts, p.nseg() * (int64_t)p.nb * p.sort_tiles() * 4, t) &&
            alloc(&w.stats, 2 * 8, t);
  if (ok && (lsh::attend_mfma_supported(p) || lsh::attend_variant_mfma_supported(p)))
    ok = alloc(&w.knorm, p.n_token_heads() * 4, t);
  if (ok && lsh::hash_mfma_supported(p)) {
    const int64_t hp = lsh::hash_half_pad(p);
    if (hipDeviceGetAttribute(&w.hash.n_cu, hipDeviceAttributeMultiprocessorCount, h->device) !=
            hipSuccess ||
        w.hash.n_cu < 1) {
      (void)hipGetLastError();
      w.hash.n_cu = 1;
    }
    ok = alloc(&w.hash.rh, (int64_t)p.R * hp * p.d * 2, t) &&
         alloc(&w.hash.rt, (int64_t)p.R * p.half() * p.d * 4, t) &&
         alloc(&w.hash.bounds, (4 * (int64_t)p.R + 2) * 4, t) &&
         alloc(&w.hash.queue_a, rows * 16, t) && alloc(&w.hash.queue_b, rows * 8, t) &&
         alloc(&w.hash.x16, p.n_token_heads() * p.d * 2, t) &&
         alloc(&w.hash.xnorm, p.n_token_heads() * 8, t);
  }
  if (ok && (p.flags & LSH_ATTN_FLAG_DEDUP)) ok = alloc(&w.inv, rows * 4, t);
  if (ok && (p.flags & LSH_ATTN_FLAG_SEPARATE_GATHER))
    ok = alloc(&w.qk_sorted, rows * p.d * esize, t) && alloc(&w.v_sorted, rows * p.d * esize, t);
  if (ok && (p.flags & LSH_ATTN_FLAG_BACKWARD)) {
    lsh::BwdWorkspace& b = h->bw;
    ok = (lsh::attend_mfma_supported(p) ? alloc(&b.od, rows * 4, t)
                                        : alloc(&b.o32, p.nseg() * p.o_seg_rows() * p.d * 4, t)) &&
         alloc(&b.lse, rows * 4, t) &&
         alloc(&b.w, rows * 4, t) && alloc(&b.cq, p.n_token_heads() * 4, t) &&
         alloc(&b.wself, p.n_token_heads() * 4, t) &&
         alloc(&b.dq, rows * p.d * (lsh::bwd_rows_half(p) ? 2 : 4), t) &&
         (lsh::attend_mfma_supported(p) || alloc(&b.dk, rows * p.d * 4, t)) &&
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
// null; x16_ready: the projection already prepared the hash's fp16 copy.
int forward_body(lsh_attn_s* h, const void* qk, const void* v, const float* rotations, void* out,
                 float* lse, int32_t* buckets, int32_t* perm, hipStream_t s, hipEvent_t* ev,
                 bool x16_ready) {
  const lsh::Problem& p = h->p;
  auto mark = [&](int j) {
    if (ev) hipEventRecord(ev[j], s);
  };
  lsh::Workspace& w = h->ws;
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
                                ev ? ev[1] : nullptr, ev ? ev[2] : nullptr, x16_ready);
    } else {
      if (w.knorm) e = lsh::launch_key_norms(p, qk, w.knorm, s);
      mark(1);
      e = lsh::launch_hash_exact(p, qk, rotations, w.buckets, buckets, s);
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
  if (e == hipSuccess) e = lsh::launch_combine(p, w.o, lsh::round_outputs_half(p), ls, v, out, s);
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
  return forward_body(h, qk, v, rotations, out, lse, buckets, perm, s, next_events(h, false),
                      false);
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
  if (ev) hipEventRecord(ev[8], s);
  bool x16_ready = false;
  const hipError_t e = lsh::launch_project(h->p, model_dim, x, w_qk, w_v, qk, v, h->ws.hash,
                                           h->ws.knorm, &x16_ready, s);
  if (ev) hipEventRecord(ev[9], s);
  if (e != hipSuccess) return LSH_ATTN_ERR_HIP;
  return forward_body(h, qk, v, rotations, out, lse, buckets, perm, s, ev, x16_ready);
}

int lsh_attn_backward(lsh_attn_t h, const void* qk, const void* v, const int32_t* perm,
                      const void* dout, void* dqk, void* dv, void* stream) {
  if (!h || !qk || !v || !perm || !dout || !dqk || !dv) return LSH_ATTN_ERR_INVALID_ARG;
  const lsh::Problem& p = h->p;
  if (!(p.flags & LSH_ATTN_FLAG_BACKWARD)) return LSH_ATTN_ERR_UNSUPPORTED;
  if (!aligned16(qk) || !aligned16(v) || !aligned16(dout) || !aligned16(dqk) || !aligned16(dv))
    return LSH_ATTN_ERR_INVALID_ARG;
  if (!on_device(h)) return LSH_ATTN_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  h->last_stream = s;
  const bool timing = h->btimed < h->timing_capacity;
  const hipEvent_t* ev =
      timing ? &h->bevents[(size_t)h->btimed * (LSH_ATTN_N_BWD_STAGES + 1)] : nullptr;
  if (timing) ++h->btimed;
  hipError_t e = lsh::launch_backward(p, qk, v, perm, dout, dqk, dv, h->ws.knorm, h->bw, s, ev);
  if (e == hipSuccess) e = hipGetLastError();
  return e == hipSuccess ? LSH_ATTN_OK : LSH_ATTN_ERR_HIP;
}

int lsh_attn_get_stats(lsh_attn_t h, lsh_attn_stats_t* stats) {
  if (!h || !stats) return LSH_ATTN_ERR_INVALID_ARG;
  unsigned long long host[2] = {0, 0};
  if (hipStreamSynchronize(h->last_stream) != hipSuccess ||
      hipMemcpy(host, h->ws.stats, sizeof(host), hipMemcpyDeviceToHost) != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  stats->n_exact_rescored = (int64_t)host[0];
  stats->n_full_fallback = (int64_t)host[1];
  return LSH_ATTN_OK;
}

static void destroy_events(lsh_attn_s* h) {
  for (hipEvent_t e : h->events) hipEventDestroy(e);
  for (hipEvent_t e : h->bevents) hipEventDestroy(e);
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
  if (switched) hipSetDevice(prev);
  delete h;
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return LSH_ATTN_ERR_HIP;
  }
  return LSH_ATTN_OK;
}

const char* lsh_attn_strerror(int status) {
  switch (status) {
    case LSH_ATTN_OK: return "ok";
    case LSH_ATTN_ERR_INVALID_ARG: return "invalid argument";
    case LSH_ATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case LSH_ATTN_ERR_OUT_OF_MEMORY: return "out of device memory";
    case LSH_ATTN_ERR_HIP: return "HIP runtime or launch error";
    default: return "unknown status";
  }
}

}  // extern "C"
