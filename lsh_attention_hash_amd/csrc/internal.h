// internal.h -- shared declarations of the HIP library (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lsh_attn.h"

namespace lsh {

// Value of the logit a query gives its own key, and the logsumexp of a round
// in which it sees nothing else. Exactly representable in fp32.
constexpr float kSelfLogit = -1.0e5f;

// One wave is 64 lanes on CDNA.
constexpr int kWave = 64;

// Elements of one (segment, tile) in the sort's histogram and scatter phases.
constexpr int kSortTile = 1024;

// Rows of padding after each segment's per-round outputs. With L a power of
// two the rounds of one position would otherwise lie a power of two apart,
// and the round combination's loads of them would meet in one DRAM bank.
constexpr int kORowPad = 17;

struct Problem {
  int B, H, L, d, nb, R, m, causal, dtype, out_dtype, flags;
  int64_t nbh() const { return (int64_t)B * H; }
  int64_t nseg() const { return nbh() * R; }           // (batch, head, round) segments
  int64_t n_token_heads() const { return nbh() * L; }
  int64_t n_rows() const { return nseg() * L; }        // (segment, position) pairs
  int64_t o_seg_rows() const { return (int64_t)L + kORowPad; }  // o rows per segment
  int half() const { return nb / 2; }
  int sort_tiles() const { return (L + kSortTile - 1) / kSortTile; }
};

// Scratch of the matrix-core hash (hash_mfma.hip).
struct HashScratch {
  _Float16* rh = nullptr;     // [R, half_pad, d] fp16 rotations, transposed, zero-padded
  float* rt = nullptr;        // [R, half, d] fp32 rotations, transposed (exact re-scoring)
  unsigned* bounds = nullptr; // [R][column tiles] float4 partial norm maxima of the
                              // rotation, then the counts of queues A and B
  void* queue_a = nullptr;    // [R * N] two-candidate re-score entries (16 B)
  void* queue_b = nullptr;    // [R * N] all-column re-score entries (8 B)
  void* xnorm = nullptr;      // [N] float2 bounds of |x16| and |x - x16| (x16: qk in fp16)
  int n_cu = 0;               // compute units of the handle's device
  int per_cu = 0;             // resident hash workgroups per CU (0: not yet queried)
  bool proj_attr = false;     // the projection kernel's LDS attribute is set
};

// Device workspace owned by a handle. Per-round arrays are [seg, L(, d)] with
// seg = (b * H + h) * R + r, i.e. the [B, H, R, L] layout of the ABI.
struct Workspace {
  uint16_t* buckets = nullptr;     // [seg, L]
  int32_t* perm = nullptr;         // [seg, L] sorted slot -> position
  int32_t* inv = nullptr;          // [seg, L] position -> sorted slot (de-duplicated union only)
  void* o = nullptr;               // [seg, L + kORowPad, d] per-round outputs at original positions
                                   // (fp16, or fp32 with the fp32 flag / plain kernel)
  float* lse = nullptr;            // [seg, L]
  uint32_t* sort_counts = nullptr; // [seg, tiles, nb] counts, then their running sums;
                                   // [seg, nb] totals; [seg, nb] first slots
  void* qk_sorted = nullptr;       // [seg, L, d] (separate-gather mode only)
  void* v_sorted = nullptr;        // [seg, L, d]
  unsigned long long* stats = nullptr;  // [4] exact rescored, full fallback (last forward);
                                        // fp16 limit hits of forward / backward rows (since
                                        // the last lsh_attn_get_stats)
  float* knorm = nullptr;          // [B*H*L] squared qk row norms (matrix-core attention)
  HashScratch hash;                     // matrix-core hash only
};

// Backward workspace (allocated with LSH_ATTN_FLAG_BACKWARD), fp32:
struct BwdWorkspace {
  float* o32 = nullptr;  // [seg, L + kORowPad, d] recomputed per-round rows (plain path)
  float* od = nullptr;   // [seg, L] dout . o_r per query (matrix-core path)
  float* lse = nullptr;  // [seg, L] recomputed per-round logsumexps
  float* w = nullptr;    // [seg, L] round weights of the combination
  float* cq = nullptr;   // [B*H, L] dout . out
  float* wself = nullptr;  // [B*H, L] summed weight of the self-only rounds (matrix-core path)
  float* dq = nullptr;   // [seg, L, d] per-round dq at original positions (matrix-core
                         // path: dq plus the normalised key gradient, dqk per round;
                         // fp16 when bwd_rows_half)
  float* dk = nullptr;   // [seg, L, d] per-round d(unit key) (plain path)
  float* dv = nullptr;   // [seg, L, d] per-round dv (fp16 when bwd_rows_half)
};

// Kernel launchers (each defined next to its kernels). All enqueue on `s` and
// return hipGetLastError().
// exact fp64 hash of every row (fp32 inputs, or shapes the matrix-core hash
// does not cover)
hipError_t launch_hash_exact(const Problem& p, const void* qk, const float* rot,
                             uint16_t* buckets, int32_t* buckets_out, hipStream_t s);
int hash_half_pad(const Problem& p);
bool hash_mfma_supported(const Problem& p);
// after_prep / after_main (may be null) are recorded once the preparation
// kernels and the projection kernel are enqueued
// knorm (may be null): receives the squared norm of every qk row (bf16
// inputs, d = 64 or 128), which the matrix-core attention uses
hipError_t launch_hash_mfma(const Problem& p, const void* qk, const float* rot, HashScratch& hs,
                            uint16_t* buckets, int32_t* buckets_out, unsigned long long* stats,
                            float* knorm, hipStream_t s, hipEvent_t after_prep,
                            hipEvent_t after_main, bool norms_ready = false);
// norms_ready: the projection already wrote hs.xnorm and knorm for qk
// the shared-QK and value projections of x (project.hip); on the matrix-core
// path also the hash's norm bounds of the qk rows and knorm
// (*norms_ready = true)
bool project_mfma_supported(const Problem& p, int model_dim);
hipError_t launch_project(const Problem& p, int model_dim, const void* x, const void* w_qk,
                          const void* w_v, void* qk, void* v, HashScratch& hs, float* knorm,
                          bool* norms_ready, hipStream_t s);
// squared norms of the qk rows alone (when the matrix-core hash does not run)
hipError_t launch_key_norms(const Problem& p, const void* qk, float* knorm, hipStream_t s);
hipError_t launch_sort(const Problem& p, const uint16_t* buckets, uint32_t* counts,
                       int32_t* perm, hipStream_t s);
hipError_t launch_gather(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                         void* qk_sorted, void* v_sorted, hipStream_t s);
// buckets [seg, L] at original positions (read by the same-bucket variant),
// inv [seg, L] (read by the de-duplicated union; may be null otherwise)
hipError_t launch_attend(const Problem& p, const void* qk, const void* v, const void* qk_sorted,
                         const void* v_sorted, const int32_t* perm, const float* knorm,
                         const uint16_t* buckets, const int32_t* inv, float* o, float* lse,
                         hipStream_t s);
// the variant readings on matrix cores (bf16, chunk_len 64, d in {64, 128};
// with DEDUP at most 8 rounds): fp32 per-round rows
bool attend_variant_mfma_supported(const Problem& p);
hipError_t launch_attend_variant_mfma(const Problem& p, const void* qk, const void* v,
                                      const int32_t* perm, const float* knorm,
                                      const uint16_t* buckets, const int32_t* inv, void* o,
                                      float* lse, hipStream_t s);
// the same kernels in the backward's recomputation form: od [seg, L] receives
// dout . o_r per query (dout . v_i for a query that saw only itself), lse the
// per-round logsumexps
hipError_t launch_attend_variant_dot(const Problem& p, const void* qk, const void* v,
                                     const int32_t* perm, const float* knorm, const void* dout,
                                     const uint16_t* buckets, const int32_t* inv, float* od,
                                     float* lse, hipStream_t s);
// inv[seg, perm[seg, s]] = s
hipError_t launch_inverse_perm(const Problem& p, const int32_t* perm, int32_t* inv, hipStream_t s);
// the plain chunk attention (any shape, every variant reading) with fp32
// per-round rows o [seg, o_seg_rows, d] and lse [seg, L]; buckets [seg, L]
// read with SAME_BUCKET, inv with DEDUP
hipError_t launch_attend_plain(const Problem& p, const void* qk, const void* v,
                               const int32_t* perm, const uint16_t* buckets, const int32_t* inv,
                               float* o, float* lse, hipStream_t s);
// bf16, chunk_len 64, d in {64, 128}: the default reading, and the unit-query
// and same-bucket readings with the gather fused
bool attend_mfma_supported(const Problem& p);
// buckets [seg, L]: read with LSH_ATTN_FLAG_SAME_BUCKET (may be null otherwise)
template <typename OT>
hipError_t launch_attend_mfma(const Problem& p, const void* qk, const void* v,
                              const void* qk_sorted, const void* v_sorted, const int32_t* perm,
                              const float* knorm, const uint16_t* buckets, OT* o, float* lse,
                              hipStream_t s);
// the per-round attention of the backward: lse as above, and per query the
// scalar dout . o_r in od [seg, L] instead of the rows; the unit-query and
// same-bucket readings as in the forward (buckets [seg, L], read with
// SAME_BUCKET)
hipError_t launch_attend_mfma_dot(const Problem& p, const void* qk, const void* v,
                                  const int32_t* perm, const float* knorm, const void* dout,
                                  const uint16_t* buckets, float* od, float* lse, hipStream_t s);
// o is fp16 when o_half, else fp32; v (the input values) supplies the rows of
// rounds in which a query saw only itself
// at_limit: incremented once per (position, 8 dims) piece whose fp16
// per-round rows reached the fp16 limit (+-65504)
hipError_t launch_combine(const Problem& p, const void* o, bool o_half, const float* lse,
                          const void* v, void* out, unsigned long long* at_limit,
                          hipStream_t s);

// gradients of qk and v given dout, at the permutations perm of a forward
// ev (may be null): 5 events, recorded before the recomputation and after
// each of its 4 stages (recomputation, rows, gradient products, reduction);
// at_limit: as for launch_combine, for the fp16 per-round gradient rows.
// Variant readings: buckets [seg, L] int32, the forward's bucket ids (read
// with SAME_BUCKET, may be null otherwise), copied to bk16 [seg, L]; inv
// [seg, L] receives the inverse permutations (DEDUP).
hipError_t launch_backward(const Problem& p, const void* qk, const void* v, const int32_t* perm,
                           const int32_t* buckets, const void* dout, void* dqk, void* dv,
                           float* knorm, uint16_t* bk16, int32_t* inv, BwdWorkspace& b,
                           unsigned long long* at_limit, hipStream_t s, const hipEvent_t* ev);

// the per-round gradient products on matrix cores (bwd_mfma_supported
// shapes): b.dq receives dqk per round (dq and the normalised dkhat), b.dv dv;
// buckets [seg, L] read with SAME_BUCKET
hipError_t launch_backward_mfma(const Problem& p, const void* qk, const void* v,
                                const int32_t* perm, const void* dout, const float* knorm,
                                const uint16_t* buckets, BwdWorkspace& b, hipStream_t s);

// the per-round gradient products of the look-ahead and de-duplicated
// readings on matrix cores (attend_variant_mfma_supported shapes): fp32 rows
// b.dq (dq, or the unit query's with NORM_QUERIES), b.dk (dkhat), b.dv, as the
// plain products write them; buckets [seg, L] read with SAME_BUCKET, inv
// [seg, L] with DEDUP
hipError_t launch_backward_var_mfma(const Problem& p, const void* qk, const void* v,
                                    const int32_t* perm, const void* dout, const float* knorm,
                                    const uint16_t* buckets, const int32_t* inv,
                                    BwdWorkspace& b, hipStream_t s);

// The variant readings (flags); the default matrix-core attention takes none
// of them (attend_variants.hip does).
constexpr int kVariantFlags = LSH_ATTN_FLAG_LOOK_AHEAD | LSH_ATTN_FLAG_SAME_BUCKET |
                              LSH_ATTN_FLAG_NORM_QUERIES | LSH_ATTN_FLAG_DEDUP;

// Per-round outputs are kept in fp16 on the matrix-core path unless the
// caller asks for fp32.
// Kernel attributes (the LDS size above 64 KiB) are set once per device:
// `done` holds one flag per device index; past kMaxDevices the attribute is
// set on every call (setting it again is harmless).
constexpr int kMaxDevices = 64;
inline bool first_on_device(bool (&done)[kMaxDevices]) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return true;
  }
  if (dev < 0 || dev >= kMaxDevices) return true;
  if (done[dev]) return false;
  done[dev] = true;
  return true;
}

inline bool round_outputs_half(const Problem& p) {
  return (attend_mfma_supported(p) || attend_variant_mfma_supported(p)) &&
         !(p.flags & LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS);
}

// The backward's products run on matrix cores on the matrix-core attention's
// shapes for the default reading and the unit-query and same-bucket readings;
// the look-ahead and de-duplicated readings take the plain kernels.
inline bool bwd_mfma_supported(const Problem& p) {
  return attend_mfma_supported(p) &&
         !(p.flags & (LSH_ATTN_FLAG_LOOK_AHEAD | LSH_ATTN_FLAG_DEDUP));
}
// The backward's recomputation runs on matrix cores, reduced to dout . o_r per
// query (no per-round rows), wherever a matrix-core forward kernel takes the
// reading: the default kernel with the matrix-core products, the variant
// kernel before the plain products (look-ahead, de-duplication).
inline bool bwd_recompute_dot(const Problem& p) {
  return bwd_mfma_supported(p) || attend_variant_mfma_supported(p);
}

// The backward's per-round gradient rows (dqk_r, dv_r) on the matrix-core path
// are kept in fp16 under the same rule; otherwise fp32.
inline bool bwd_rows_half(const Problem& p) {
  return bwd_mfma_supported(p) && !(p.flags & LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS);
}

}  // namespace lsh
