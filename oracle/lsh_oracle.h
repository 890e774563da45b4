/*
 * lsh_oracle.h -- plain, slow fp64 CPU definition of Reformer shared-QK LSH
 * self-attention (forward, and its backward at fixed buckets).
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline may load or call this library. The product path (the HIP library
 * and its Python binding) never links, imports or calls it, and it shares no
 * code, header, constant or helper with that path.
 *
 * Sources for each step (the pages are web summaries of the Reformer paper):
 *   [TT] Reformer summary, p2.ttnews.xyz/a/5dd41cfcdc9b5e51a0429126
 *        sections: LSH (hash of a vector with a random matrix R of size
 *        [dimension, b/2], h(x) = argmax of the concatenation [xR; -xR]);
 *        LSH attention (sort by bucket, then by position inside a bucket; cut
 *        the sorted sequence into groups of m and attend inside them);
 *        multi-round LSH (several independent hash functions);
 *        self-mask for shared QK (no attention to oneself unless nothing else
 *        can be attended to).
 *   [DT] Reformer overview, www.dtcms.com/a/488796.html, section 2.1
 *        "key steps": unit-normalised keys, multiple projection rounds, each
 *        query also looks at the neighbouring group; "math" paragraph: the
 *        scaled softmax with 1/sqrt(d_k) and a mask; section 2.3: the
 *        reversible block and the chunked feed-forward layer.
 * Where the pages leave a step open, the reading taken is stated at the step
 * in lsh_oracle.c.
 *
 * Layouts (row-major, contiguous):
 *   qk, v, out        [B, H, L, d]            float64
 *   rotations         [n_rounds, d, n_buckets/2] float64 (unused when n_buckets == 1)
 *   buckets, perm, inv [B, H, n_rounds, L]    int32
 *   margin            [B, H, n_rounds, L]     float64 (largest minus second-largest of
 *                                              the concatenated projection)
 *   o                 [B, H, n_rounds, L, d]  float64, indexed by ORIGINAL position
 *   lse               [B, H, n_rounds, L]     float64, indexed by original position
 * perm maps a sorted slot to the position it holds; inv is its inverse.
 * All functions return 0 on success and a negative value on a bad config.
 */
#ifndef LSH_ORACLE_H
#define LSH_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, heads, seq_len, head_dim;
  int32_t n_buckets;  /* 1, or even >= 2 */
  int32_t n_rounds;   /* >= 1 */
  int32_t chunk_len;  /* >= 1, divides seq_len */
  int32_t causal;     /* 0 or 1 */
  int32_t variant;    /* 0, or LSH_ORACLE_* bits below */
} lsh_oracle_config;

/* Variant readings (bits of variant; 0 is the default reading). Each is a
 * reading the pages also support:
 *   LOOK_AHEAD   the window also holds the next chunk ([DT] section 2.1: a
 *                query looks at the neighbouring groups, one before and one
 *                after);
 *   SAME_BUCKET  inside the window only keys of the query's own bucket in that
 *                round are attendable ([DT] math paragraph: the mask M keeps
 *                positions of the same bucket);
 *   NORM_QUERIES queries are unit-normalised as well as keys ([DT] section
 *                2.1: keys and queries are normalised to unit vectors);
 *   DEDUP        a key that several rounds give a query counts once: the
 *                query attends to the union of its rounds' key sets ([2K]
 *                www.2kiu.com/news/5253576/ section 2.2: the final candidate
 *                set is the de-duplicated union over rounds).
 * The backward supports the default reading only. */
#define LSH_ORACLE_LOOK_AHEAD 1
#define LSH_ORACLE_SAME_BUCKET 2
#define LSH_ORACLE_NORM_QUERIES 4
#define LSH_ORACLE_DEDUP 8

/* Logit given to a query's own key; also the logsumexp of a round in which the
 * query can attend to nothing but itself. */
#define LSH_ORACLE_SELF_LOGIT (-1.0e5)

int lsh_oracle_check(const lsh_oracle_config* cfg);

int lsh_oracle_hash(const lsh_oracle_config* cfg, const double* qk, const double* rotations,
                    int32_t* buckets, double* margin);

int lsh_oracle_sort(const lsh_oracle_config* cfg, const int32_t* buckets, int32_t* perm,
                    int32_t* inv);

/* buckets [B, H, R, L] (original positions) is read only with SAME_BUCKET and
 * may be NULL otherwise. With DEDUP, o and lse are the rounds' outputs with
 * each logit lowered by log N_ij (N_ij = the number of rounds that give key j
 * to query i), whose combination is the union's attention. */
int lsh_oracle_attend(const lsh_oracle_config* cfg, const double* qk, const double* v,
                      const int32_t* perm, const int32_t* buckets, double* o, double* lse);

int lsh_oracle_combine(const lsh_oracle_config* cfg, const double* o, const double* lse,
                       double* out);

/* Whole forward. buckets_override (nullable) replaces the hash step's buckets;
 * margin is still computed from the projections when rotations are given.
 * With DEDUP, out is computed from the union of the rounds' key sets directly,
 * and lse is that of lsh_oracle_attend. */
int lsh_oracle_forward(const lsh_oracle_config* cfg, const double* qk, const double* v,
                       const double* rotations, const int32_t* buckets_override,
                       double* out, double* lse, int32_t* buckets, int32_t* perm,
                       double* margin);

/* Backward at fixed permutations: dqk, dv [B, H, L, d] from dout [B, H, L, d]
 * (gradient of a loss with respect to out); perm [B, H, R, L] as from forward;
 * buckets [B, H, R, L] as from forward, needed with SAME_BUCKET (-12 if NULL
 * then), else may be NULL. Every variant reading. */
int lsh_oracle_backward(const lsh_oracle_config* cfg, const double* qk, const double* v,
                        const int32_t* perm, const int32_t* buckets, const double* dout,
                        double* dqk, double* dv);

/* Upper bounds of the absolute values of the backward's terms, summed as the
 * backward sums them (test infrastructure for error bounds): |dv| <= mdv and
 * |dqk| <= mdqk elementwise; see lsh_oracle.c. Arguments as for the backward. */
int lsh_oracle_backward_magnitudes(const lsh_oracle_config* cfg, const double* qk,
                                   const double* v, const int32_t* perm, const int32_t* buckets,
                                   const double* dout, double* mdqk, double* mdv);

/* The shared-QK and value projections of a layer input ([TT] shared-QK section:
 * one linear map gives queries and keys, a second one the values):
 *   qk[b, h, i, e] = sum_k x[b, i, k] w_qk[h * d + e, k],  v likewise with w_v.
 * x [B, L, model_dim]; w_qk, w_v [H * d, model_dim] (the weight of a linear
 * layer from model_dim to H * d features); qk, v [B, H, L, d]. */
int lsh_oracle_project(const lsh_oracle_config* cfg, int64_t model_dim, const double* x,
                       const double* w_qk, const double* w_v, double* qk, double* v);

/* The chunked feed-forward layer of the reversible block ([DT] section 2.3,
 * chunked feed-forward; [TT] reversible Transformer and "FF layer chunking"
 * sections): the rows (positions) are cut into chunks of chunk_rows (the last
 * one shorter when rows is not a multiple), each chunk goes through the
 * feed-forward on its own, and the outputs are concatenated:
 *   hidden[i, j] = max(0, sum_k y1[i, k] w1[j, k] + b1[j])
 *   y2[i, e]     = x2[i, e] + sum_j hidden[i, j] w2[e, j] + b2[e]
 * y1, x2, y2 [rows, d_model]; w1 [d_ff, d_model] and w2 [d_model, d_ff] (the
 * weights of linear layers d_model -> d_ff and back); b1 [d_ff], b2 [d_model].
 * x2 may be NULL (no residual; y2 is then the feed-forward alone). hidden, if
 * not NULL, receives [rows, d_ff]. Returns -13 on bad sizes. */
int lsh_oracle_ffn(int64_t rows, int64_t d_model, int64_t d_ff, int64_t chunk_rows,
                   const double* y1, const double* w1, const double* b1, const double* w2,
                   const double* b2, const double* x2, double* y2, double* hidden);

/* Output rows for a sample of (b, h, i), given every round's perm (and buckets,
 * as for lsh_oracle_attend): rows[k] = (b * H + h) * L + i; out_rows [n_rows, d];
 * lse_rows [n_rows, n_rounds]. */
int lsh_oracle_attend_rows(const lsh_oracle_config* cfg, const double* qk, const double* v,
                           const int32_t* perm, const int32_t* buckets, int64_t n_rows,
                           const int64_t* rows, double* out_rows, double* lse_rows);

#ifdef __cplusplus
}
#endif
#endif
