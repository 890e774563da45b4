/*
 * lsh_attn.h -- C ABI of the MI355X (gfx950) Reformer shared-QK LSH
 * self-attention forward pass.
 *
 * What one forward computes (the Reformer summary at p2.ttnews.xyz, sections
 * on LSH, LSH attention, multi-round LSH and the shared-QK self-mask; the
 * overview at www.dtcms.com/a/488796.html, section 2.1):
 *   1. hash: for every position i and round r, bucket = argmax([x R_r; -x R_r])
 *      where x is the shared query/key vector and R_r a [d, n_buckets/2]
 *      rotation; lowest index on exact ties;
 *   2. sort: positions ordered by (bucket, position) per (batch, head, round);
 *   3. gather: qk and v rows in sorted order;
 *   4. chunked attention: the sorted sequence is cut into chunks of chunk_len;
 *      a query attends to its chunk and the previous one (none before chunk 0),
 *      with unit-normalised keys, logits (q . k/|k|) / sqrt(d), an optional
 *      causal mask on original positions, and a self-mask: its own key gets
 *      logit -1e5, so it is used only when nothing else is attendable. Each
 *      round yields an output row o_r(i) and its logsumexp lse_r(i);
 *   5. unsort and combine: out(i) = sum_r softmax_r(lse_r(i)) o_r(i).
 *
 * Conventions for every entry point:
 *   - tensor arguments are DEVICE pointers on the current HIP device,
 *     contiguous, row-major, and owned by the caller; the library never frees
 *     or retains them past the call;
 *   - the config and handle pointers are HOST pointers;
 *   - `stream` is a hipStream_t passed as void* (NULL = the legacy default
 *     stream); all device work is enqueued on it and the call returns without
 *     waiting for the device;
 *   - every function returns a lsh_attn_status_t; nothing is thrown across
 *     the ABI. lsh_attn_strerror() maps a status to a static string.
 */
#ifndef LSH_ATTN_H
#define LSH_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct lsh_attn_s* lsh_attn_t;

typedef enum {
  LSH_ATTN_FP32 = 0,
  LSH_ATTN_BF16 = 1
} lsh_attn_dtype_t;

typedef enum {
  LSH_ATTN_OK = 0,
  LSH_ATTN_ERR_INVALID_ARG = 1,   /* null required pointer, bad sizes, bad flag */
  LSH_ATTN_ERR_UNSUPPORTED = 2,   /* valid but not implemented (head_dim, dtype) */
  LSH_ATTN_ERR_OUT_OF_MEMORY = 3, /* workspace allocation failed in create */
  LSH_ATTN_ERR_HIP = 4,           /* a HIP runtime call or kernel launch failed */
  LSH_ATTN_ERR_WORKSPACE_TOO_LARGE = 5  /* lsh_attn_forward_static: the problem's workspace
                                           exceeds LSH_ATTN_STATIC_SCRATCH_BYTES */
} lsh_attn_status_t;

/* Flags (bit set in lsh_attn_config_t.flags). */
enum {
  /* Run the gather as its own kernel that writes sorted copies of qk and v
   * (workspace grows by 2 * n_rounds * |qk|). By default the chunk-attention
   * kernel reads rows through the permutation itself. Results are identical. */
  LSH_ATTN_FLAG_SEPARATE_GATHER = 1,
  /* Keep the per-round outputs (and the backward's per-round gradient rows)
   * in fp32 between the attention and the combine step. By default the
   * matrix-core path (bf16 inputs) keeps them in fp16, which halves that
   * traffic; fp16 holds at most +-65504 and larger values are clamped there,
   * so inputs whose |v| (or, in the backward, |dout| |v| or |dout| |qk|)
   * reaches that magnitude need this flag. lsh_attn_get_stats counts the
   * values that reached the limit. */
  LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS = 2,
  /* Also allocate the workspace of lsh_attn_backward, per position and round:
   * on the matrix-core shapes (bf16, chunk_len 64, head_dim 64 or 128) 2 rows
   * of head_dim (fp16, or fp32 with LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS), or 3
   * fp32 rows with LOOK_AHEAD or DEDUP, plus 12 bytes; on the other shapes 4
   * fp32 rows plus 8 bytes. Plus 8 bytes per position. */
  LSH_ATTN_FLAG_BACKWARD = 4,
  /* Variant readings of the window and the combination, each one the pages
   * also describe (the default, all off, is the previous chunk and the chunk
   * itself, no bucket mask, raw queries, rounds combined as a multiset):
   * the window also holds the next chunk (Reformer overview at
   * www.dtcms.com/a/488796.html, section 2.1: one neighbouring group before
   * and one after); the last chunk has none. */
  LSH_ATTN_FLAG_LOOK_AHEAD = 8,
  /* inside the window only keys in the query's own bucket of that round are
   * attendable (the same page's mask M of same-bucket positions) */
  LSH_ATTN_FLAG_SAME_BUCKET = 16,
  /* queries are unit-normalised as well as keys (same page, section 2.1) */
  LSH_ATTN_FLAG_NORM_QUERIES = 32,
  /* a key given to a query by several rounds counts once: the query attends
   * to the union of its rounds' key sets (www.2kiu.com/news/5253576/, section
   * 2.2: the de-duplicated union over rounds). Computed per round with each
   * logit lowered by log N (N = the number of rounds that give the pair);
   * the lse output holds those per-round values. */
  LSH_ATTN_FLAG_DEDUP = 64
};

typedef struct {
  int32_t batch, heads, seq_len, head_dim; /* qk, v, out: [batch, heads, seq_len, head_dim] */
  int32_t n_buckets;  /* 1 (hash skipped: every position in bucket 0), or even in [2, 65536] */
  int32_t n_rounds;   /* >= 1 independent hash rounds */
  int32_t chunk_len;  /* >= 1 and divides seq_len; 64 is the tuned value */
  int32_t causal;     /* 0 or 1 */
  int32_t dtype;      /* lsh_attn_dtype_t of qk and v */
  int32_t out_dtype;  /* lsh_attn_dtype_t of out; arithmetic is fp32 (fp64 for hash ties) */
  int32_t flags;      /* LSH_ATTN_FLAG_* */
} lsh_attn_config_t;

/*
 * Create a handle for one problem shape. Validates the config and allocates
 * the device workspace on the current device (hipMalloc): bucket ids, the
 * permutation, per-round outputs and logsumexps, sort histograms, and (with
 * LSH_ATTN_FLAG_SEPARATE_GATHER) the sorted copies. The handle owns it.
 * Errors: INVALID_ARG for a null pointer, non-positive sizes, seq_len > 2^24,
 * seq_len % chunk_len != 0, an odd n_buckets > 1, n_buckets > 65536,
 * causal not 0/1, unknown flags; UNSUPPORTED for head_dim not in {64, 128},
 * chunk_len > 256, or a dtype outside the enum; OUT_OF_MEMORY if the
 * workspace cannot be allocated; HIP if no device is current.
 * On error *handle is set to NULL and nothing is left allocated.
 */
int lsh_attn_create(const lsh_attn_config_t* cfg, lsh_attn_t* handle);

/*
 * Enqueue one forward pass on `stream`.
 *   qk        [B, H, L, d]          dtype     shared query/key vectors (read only)
 *   v         [B, H, L, d]          dtype     values (read only)
 *   rotations [n_rounds, d, n_buckets/2] fp32 random rotations (read only);
 *                                          may be NULL only when n_buckets == 1
 *   out       [B, H, L, d]          out_dtype combined output (written)
 *   lse       [B, H, n_rounds, L]   fp32, nullable: per-round logsumexp at each
 *                                          ORIGINAL position (-1e5 for a round in
 *                                          which the position saw only itself)
 *   buckets   [B, H, n_rounds, L]   int32, nullable: bucket ids
 *   perm      [B, H, n_rounds, L]   int32, nullable: sorted slot -> position
 * qk, v and out must be 16-byte aligned. Inputs must not alias outputs.
 * NaN/Inf inputs give undefined results (not checked). One forward at a time per handle: the workspace is reused, so
 * two forwards of one handle must be ordered on the device (same stream).
 * Performs no allocation and no host/device synchronisation.
 * Errors: INVALID_ARG for a null handle or required pointer, a misaligned
 * pointer, or a current device other than the handle's; HIP when a launch
 * fails (hipGetLastError after the launches).
 */
int lsh_attn_forward(lsh_attn_t handle, const void* qk, const void* v, const float* rotations,
                     void* out, float* lse, int32_t* buckets, int32_t* perm, void* stream);

/*
 * The forward from a layer input: qk and v are first computed from x by the
 * shared-QK and the value projections (Reformer summary at p2.ttnews.xyz,
 * shared-QK section: one linear map gives both queries and keys, another the
 * values), then the forward runs on them exactly as lsh_attn_forward:
 *   qk[b, h, i, e] = sum_k x[b, i, k] w_qk[h * head_dim + e, k]   (v: w_v)
 *   x        [B, L, model_dim]            dtype (read only)
 *   w_qk, w_v [H * head_dim, model_dim]   dtype (read only): the weights of
 *            linear layers from model_dim to H * head_dim features
 *   qk, v    [B, H, L, head_dim]          dtype (written; caller-owned, for
 *            a later backward), rounded from fp32 sums
 *   rotations, out, lse, buckets, perm    as for lsh_attn_forward
 * On the matrix-core path (bf16, head_dim 64 or 128, model_dim a multiple of
 * 32, and the hash on matrix cores) the projection kernel also writes the
 * hash's fp16 copy of qk and its norms, which the hash then does not recompute.
 * Device pointers, all 16-byte aligned. No allocation, no host
 * synchronisation; timing stage 7 is the projection.
 * Errors: INVALID_ARG for a null handle or pointer, model_dim < 1 (or
 * model_dim * H * head_dim > 2^31), a misaligned pointer or a current device
 * other than the handle's; HIP when a launch fails.
 */
int lsh_attn_forward_x(lsh_attn_t handle, const void* x, int32_t model_dim, const void* w_qk,
                       const void* w_v, const float* rotations, void* qk, void* v, void* out,
                       float* lse, int32_t* buckets, int32_t* perm, void* stream);

/*
 * Enqueue the backward of a forward on `stream`: the gradients of a loss with
 * respect to qk and v, given dout = dL/dout, at that forward's buckets (the
 * hash is an argmax and the sort a permutation, both piecewise constant, so
 * no gradient flows through them). The chain rule is taken through the
 * round combination, the windowed softmax, the shared-QK logits and the key
 * normalisation (Reformer summary at p2.ttnews.xyz, LSH attention and
 * multi-round sections; overview at www.dtcms.com/a/488796.html, section
 * 2.1). The per-round attention is recomputed from the permutation.
 *   qk, v     [B, H, L, d]          dtype  (read only), as passed to the forward
 *   perm      [B, H, n_rounds, L]   int32  (read only): the forward's perm output
 *   dout      [B, H, L, d]          dtype  (read only)
 *   dqk, dv   [B, H, L, d]          dtype  (written); must not alias the inputs
 * Device pointers; qk, v, dout, dqk and dv 16-byte aligned. Uses the handle's
 * backward workspace (LSH_ATTN_FLAG_BACKWARD at create) and the forward's key
 * norm buffer, so a backward and a forward of one handle must be ordered on the
 * device (same stream). Performs no allocation and no host/device
 * synchronisation. Deterministic: every output element is written once.
 * Errors: INVALID_ARG for a null handle or pointer, a misaligned pointer or a
 * current device other than the handle's, or LSH_ATTN_FLAG_SAME_BUCKET (which
 * needs the forward's bucket ids: lsh_attn_backward_buckets); UNSUPPORTED if
 * the handle was created without LSH_ATTN_FLAG_BACKWARD; HIP when a launch
 * fails.
 */
int lsh_attn_backward(lsh_attn_t handle, const void* qk, const void* v, const int32_t* perm,
                      const void* dout, void* dqk, void* dv, void* stream);

/*
 * The same backward for handles created with the variant flags: the window
 * and the logits are those of the forward's reading (look-ahead chunk,
 * same-bucket mask, unit queries, de-duplicated rounds; Reformer overview at
 * www.dtcms.com/a/488796.html, section 2.1, and www.2kiu.com/news/5253576/,
 * section 2.2). With LSH_ATTN_FLAG_NORM_QUERIES the unit query q / |q| takes
 * the same normalisation Jacobian as the unit key of that row. Unit queries and
 * the same-bucket mask run on the matrix-core path of the default reading; the
 * look-ahead and de-duplicated readings on matrix-core kernels of their own
 * (fp32 per-round gradient rows) where the forward's variant kernel takes the
 * shape (bf16, chunk_len 64, d in {64, 128}, with DEDUP at most 8 rounds), on
 * the plain kernels otherwise.
 *   buckets   [B, H, n_rounds, L]   int32  (read only): the forward's buckets
 *             output; required with LSH_ATTN_FLAG_SAME_BUCKET (INVALID_ARG if
 *             null then), may be null otherwise
 * Other arguments, workspace and errors as for lsh_attn_backward, which is
 * this call with buckets null. Uses the handle's bucket-id buffer and, with
 * LSH_ATTN_FLAG_DEDUP, its inverse-permutation buffer as scratch.
 */
int lsh_attn_backward_buckets(lsh_attn_t handle, const void* qk, const void* v,
                              const int32_t* perm, const int32_t* buckets, const void* dout,
                              void* dqk, void* dv, void* stream);

/*
 * Counters (waits for the handle's last stream):
 *   n_exact_rescored, n_full_fallback (of the last forward): hash decisions the
 *   bulk projection could not certify, settled by recomputing in fp64 the two
 *   candidate columns or every column;
 *   n_round_rows_at_fp16_limit (forwards since the previous call of this
 *   function): (position, 8 dims) pieces whose fp16 per-round output rows
 *   reached +-65504, the fp16 limit, where values are clamped. The per-round
 *   rows are kept in fp16 on the matrix-core path unless
 *   LSH_ATTN_FLAG_FP32_ROUND_OUTPUTS is set; they are convex combinations of
 *   v rows, so this stays 0 while every |v| < 65504; a nonzero count means the
 *   affected outputs are inaccurate and the handle should use the flag;
 *   n_grad_rows_at_fp16_limit (backwards since the previous call): the same
 *   for the backward's fp16 per-round gradient rows (dqk_r, dv_r), whose
 *   magnitudes grow with |dout| |v| and |dout| |qk|.
 * The two limit counters restart at 0 after each call.
 * Errors: INVALID_ARG for null pointers; HIP if a copy fails.
 */
typedef struct {
  int64_t n_exact_rescored;
  int64_t n_full_fallback;
  int64_t n_round_rows_at_fp16_limit;
  int64_t n_grad_rows_at_fp16_limit;
} lsh_attn_stats_t;
int lsh_attn_get_stats(lsh_attn_t handle, lsh_attn_stats_t* stats);

/*
 * Per-stage device timing, for diagnostics and the benchmark. When enabled,
 * each forward records a HIP event on its stream before the first stage and
 * after every stage, for at most `capacity` forwards (later forwards are not
 * timed). Events are created here (host call, no device memory).
 * Stages: 0 hash preparation (rotation copies, fp16 copy of qk; 0 ms on the
 * exact fp64 path), 1 hash projection (the matrix-core kernel, or the exact
 * kernel), 2 exact re-scoring of unsettled rows (0 ms on the exact path),
 * 3 sort, 4 gather (0 ms unless separate), 5 chunk attention, 6 combine,
 * 7 the qk/v projections of lsh_attn_forward_x (0 ms for lsh_attn_forward).
 * Errors: INVALID_ARG for a null handle or capacity < 0 (0 disables);
 * HIP if events cannot be created.
 */
#define LSH_ATTN_N_STAGES 8
int lsh_attn_set_timing(lsh_attn_t handle, int capacity);

/*
 * Sum of each stage's elapsed milliseconds over the timed forwards since the
 * last call (waits for their events), and how many forwards that was; then
 * starts a new accumulation. ms has LSH_ATTN_N_STAGES entries (host memory).
 * Errors: INVALID_ARG for null pointers or timing not enabled; HIP on event errors.
 */
int lsh_attn_get_timing(lsh_attn_t handle, double* ms, int64_t* n_forwards);

/*
 * The same for lsh_attn_backward: with timing enabled (lsh_attn_set_timing,
 * the same capacity, counted separately), each backward records an event
 * before its first stage and after every stage. Stages: 0 recomputation of the
 * per-round attention (key norms and the chunk attention at the given
 * permutation), 1 per-position round weights and dout . out, 2 the per-round
 * gradient products (dq of every query, dkhat and dv of every key), 3 the sum
 * over rounds. ms has LSH_ATTN_N_BWD_STAGES entries
 * (host memory); n_backwards receives the number of timed backwards, and the
 * accumulation restarts.
 * Errors: INVALID_ARG for null pointers or timing not enabled; HIP on event errors.
 */
#define LSH_ATTN_N_BWD_STAGES 4
int lsh_attn_get_backward_timing(lsh_attn_t handle, double* ms, int64_t* n_backwards);

/*
 * The forward of lsh_attn_forward without a handle and without any allocation,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc). Same
 * arguments, results and conventions as lsh_attn_forward, with the config
 * passed directly (host pointer); LSH_ATTN_FLAG_BACKWARD is not accepted
 * (UNSUPPORTED). The workspace comes from a static device array of
 * LSH_ATTN_STATIC_SCRATCH_BYTES that every GPU the library runs on holds
 * until the process ends; its address is looked up once per device, on the
 * first call there. Every call on one GPU shares that GPU's array, so calls
 * that overlap on one GPU (other streams, other threads) race and give
 * undefined results: order them on the device. No stage timing, and no
 * counters (lsh_attn_get_stats needs a handle). The workspace is that of a
 * handle for the same config (per-round rows, permutations, hash buffers):
 * about 61 MB for batch 4, 8 heads, L 4096, head_dim 64, 64 buckets, 2
 * rounds; larger problems need a handle.
 * Errors: those of lsh_attn_create's validation and of lsh_attn_forward,
 * UNSUPPORTED with LSH_ATTN_FLAG_BACKWARD, WORKSPACE_TOO_LARGE when the
 * problem's workspace exceeds the static array (nothing is launched).
 */
#define LSH_ATTN_STATIC_SCRATCH_BYTES ((int64_t)64 << 20)
int lsh_attn_forward_static(const lsh_attn_config_t* cfg, const void* qk, const void* v,
                            const float* rotations, void* out, float* lse, int32_t* buckets,
                            int32_t* perm, void* stream);

/* Bytes of device workspace the handle holds. INVALID_ARG for null pointers. */
int lsh_attn_workspace_bytes(lsh_attn_t handle, int64_t* bytes);

/* Free the workspace (synchronises the device first). NULL is accepted. */
int lsh_attn_destroy(lsh_attn_t handle);

/* Static, never-NULL description of a status code. */
const char* lsh_attn_strerror(int status);

/* ---------------------------------------------------------------------------
 * Chunked feed-forward: the other half of the reversible block that holds the
 * attention (Reformer overview at www.dtcms.com/a/488796.html, section 2.3:
 * y2 = x2 + FeedForward(y1), and the chunked feed-forward applied to one
 * chunk of rows at a time with the chunk outputs concatenated; the Reformer
 * summary at p2.ttnews.xyz, "FF layer chunking"). Per row i:
 *   hidden[i, :] = max(0, W1 y1[i, :] + b1)         (d_ff values)
 *   y2[i, :]     = x2[i, :] + W2 hidden[i, :] + b2   (x2 optional)
 * Rows go in chunks of chunk_rows; only one chunk's hidden rows are held
 * (chunk_rows x d_ff in the layer dtype, in the handle's workspace). A row's
 * output is bit-identical whatever the chunking.
 * Statuses and pointer conventions are those of the attention entry points.
 */
typedef struct lsh_ffn_s* lsh_ffn_t;

typedef struct {
  int64_t max_rows;   /* most rows a forward may take (>= 1) */
  int64_t chunk_rows; /* rows per chunk; 0 = all rows in one chunk */
  int32_t d_model;    /* features of y1, x2, y2 (a multiple of 8) */
  int32_t d_ff;       /* hidden features (a multiple of 8) */
  int32_t dtype;      /* lsh_attn_dtype_t of every tensor; fp32 accumulation */
} lsh_ffn_config_t;

/*
 * Create a handle and allocate the chunk's hidden buffer (hipMalloc,
 * min(chunk_rows, max_rows) x d_ff elements) on the current device.
 * Errors: INVALID_ARG for null pointers or sizes below the limits above;
 * UNSUPPORTED for a dtype outside the enum or d_model / d_ff not multiples of
 * 8 (and for shapes off the matrix-core path whose chunk exceeds 2^31
 * elements); OUT_OF_MEMORY if the buffer cannot be allocated.
 */
int lsh_ffn_create(const lsh_ffn_config_t* cfg, lsh_ffn_t* handle);

/*
 * y2 [rows, d_model] from y1 [rows, d_model], w1 [d_ff, d_model], b1 [d_ff],
 * w2 [d_model, d_ff], b2 [d_model] and x2 [rows, d_model] (NULL: no
 * residual). Device pointers; y1, w1, w2, x2 and y2 16-byte aligned. y2 may
 * alias x2 (each element is read before it is written, by the same thread);
 * it must not overlap y1. rows = 0 does nothing. The matrix-core path takes
 * bf16 with d_model and d_ff multiples of 128; the hidden rows are rounded
 * to the layer dtype between the two layers.
 * Errors: INVALID_ARG for a null handle or required pointer, misalignment,
 * rows < 0 or rows > max_rows, or a device other than the handle's;
 * HIP on a launch error.
 */
int lsh_ffn_forward(lsh_ffn_t handle, int64_t rows, const void* y1, const void* w1,
                    const void* b1, const void* w2, const void* b2, const void* x2, void* y2,
                    void* stream);

/*
 * Device timing as for the attention: with capacity > 0, each of the next
 * `capacity` forwards records an event before its first launch and after
 * every launch. lsh_ffn_get_timing sums, over the timed forwards since the
 * last call, stage 0 (the first layer, every chunk) and stage 1 (the second
 * layer) into ms[LSH_FFN_N_STAGES], stores the number of forwards and (if
 * n_chunks is not NULL) of chunks, and restarts the accumulation.
 * Errors: INVALID_ARG for null pointers or timing not enabled; HIP on event errors.
 */
#define LSH_FFN_N_STAGES 2
int lsh_ffn_set_timing(lsh_ffn_t handle, int capacity);
int lsh_ffn_get_timing(lsh_ffn_t handle, double* ms, int64_t* n_forwards, int64_t* n_chunks);

/* Bytes of device workspace (the hidden buffer). INVALID_ARG for null pointers. */
int lsh_ffn_workspace_bytes(lsh_ffn_t handle, int64_t* bytes);

/* Free the handle (synchronises the device first). NULL is accepted. */
int lsh_ffn_destroy(lsh_ffn_t handle);

#ifdef __cplusplus
}
#endif
#endif /* LSH_ATTN_H */
