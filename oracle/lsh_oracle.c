/*
 * lsh_oracle.c -- the plain fp64 CPU oracle. TEST INFRASTRUCTURE only: see
 * lsh_oracle.h for who may call it, the page sources ([TT], [DT]) and layouts.
 *
 * Every step is written the slow, literal way, one query at a time, in the
 * order the pages give the method. OpenMP only splits independent
 * (batch, head, round) segments or positions across threads; nothing is
 * blocked, fused or reordered inside a step.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off -fPIC -shared (no fast-math).
 */
#include "lsh_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

int lsh_oracle_check(const lsh_oracle_config* c) {
  if (!c) return -1;
  if (c->batch < 1 || c->heads < 1 || c->seq_len < 1 || c->head_dim < 1) return -2;
  if (c->n_rounds < 1 || c->chunk_len < 1 || c->seq_len % c->chunk_len != 0) return -3;
  if (c->n_buckets < 1 || (c->n_buckets > 1 && c->n_buckets % 2 != 0)) return -4;
  if (c->causal != 0 && c->causal != 1) return -5;
  if (c->variant < 0 || c->variant > 15) return -11;
  return 0;
}

static size_t seg_count(const lsh_oracle_config* c) {
  return (size_t)c->batch * c->heads * c->n_rounds;
}

/* ---------------------------------------------------------------------------
 * Hash, [TT] section LSH: R has size [d, b/2]; h(x) is the index of the
 * largest entry of the length-b vector [xR; -xR]. Several rounds use
 * independent R ([TT] multi-round LSH); R is shared by every batch and head
 * (the figure caption of [TT] LSH attention notes that R is shared).
 * Readings where the page is silent:
 *   - ties: the lowest index wins (exact ties only happen for x = 0 and on
 *     sets of measure zero);
 *   - n_buckets == 1: [d, b/2] is empty, every position is in bucket 0 and its
 *     margin is +inf.
 * margin = largest minus second-largest entry of [xR; -xR]; it measures how
 * close a bucket decision is to a tie.
 * ------------------------------------------------------------------------- */
int lsh_oracle_hash(const lsh_oracle_config* c, const double* qk, const double* rot,
                    int32_t* buckets, double* margin) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  const int64_t L = c->seq_len, d = c->head_dim, nb = c->n_buckets, R = c->n_rounds;
  const int64_t half = nb / 2;
  const int64_t nseg = (int64_t)seg_count(c);
  if (nb > 1 && !rot) return -6;
#pragma omp parallel
  {
    double* z = (double*)malloc(sizeof(double) * (size_t)(nb > 1 ? nb : 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t seg = 0; seg < nseg; ++seg) {
      const int64_t bh = seg / R, r = seg % R;
      const double* x_bh = qk + bh * L * d;
      for (int64_t i = 0; i < L; ++i) {
        const size_t out_idx = (size_t)(seg * L + i);
        if (nb == 1) {
          buckets[out_idx] = 0;
          if (margin) margin[out_idx] = INFINITY;
          continue;
        }
        const double* x = x_bh + i * d;
        const double* Rr = rot + r * d * half;
        /* projection xR: p_k = sum_t x_t R[t][k]; then z = [p; -p] */
        for (int64_t k = 0; k < half; ++k) {
          double p = 0.0;
          for (int64_t t = 0; t < d; ++t) p += x[t] * Rr[t * half + k];
          z[k] = p;
          z[k + half] = -p;
        }
        int64_t best = 0;
        for (int64_t k = 1; k < nb; ++k)
          if (z[k] > z[best]) best = k;
        double second = -INFINITY;
        for (int64_t k = 0; k < nb; ++k)
          if (k != best && z[k] > second) second = z[k];
        buckets[out_idx] = (int32_t)best;
        if (margin) margin[out_idx] = z[best] - second;
      }
    }
    free(z);
  }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Sort, [TT] section LSH attention: order positions by bucket, ascending, and
 * inside a bucket by position. Written as a counting sort over bucket ids that
 * visits positions in increasing order, which keeps equal buckets in position
 * order. perm[s] = position held by sorted slot s; inv[perm[s]] = s.
 * ------------------------------------------------------------------------- */
int lsh_oracle_sort(const lsh_oracle_config* c, const int32_t* buckets, int32_t* perm,
                    int32_t* inv) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  const int64_t L = c->seq_len, nb = c->n_buckets;
  const int64_t nseg = (int64_t)seg_count(c);
  int bad = 0;
#pragma omp parallel
  {
    int64_t* start = (int64_t*)malloc(sizeof(int64_t) * (size_t)(nb + 1));
#pragma omp for schedule(dynamic, 1)
    for (int64_t seg = 0; seg < nseg; ++seg) {
      const int32_t* bk = buckets + seg * L;
      int32_t* pm = perm + seg * L;
      for (int64_t b = 0; b <= nb; ++b) start[b] = 0;
      int local_bad = 0;
      for (int64_t i = 0; i < L; ++i) {
        if (bk[i] < 0 || bk[i] >= nb) { local_bad = 1; break; }
        start[bk[i] + 1] += 1;
      }
      if (local_bad) {
#pragma omp atomic write
        bad = 1;
        continue;
      }
      for (int64_t b = 0; b < nb; ++b) start[b + 1] += start[b];
      for (int64_t i = 0; i < L; ++i) pm[start[bk[i]]++] = (int32_t)i;
      if (inv) {
        int32_t* iv = inv + seg * L;
        for (int64_t s = 0; s < L; ++s) iv[pm[s]] = (int32_t)s;
      }
    }
    free(start);
  }
  return bad ? -7 : 0;
}

/* ---------------------------------------------------------------------------
 * One query of one round.
 * [TT] LSH attention: the sorted sequence is cut into chunks of m and a query
 * attends inside its chunk; [DT] 2.1 adds the neighbouring chunk. Reading
 * taken: the window of a query in chunk c is chunk c plus chunk c-1 (chunk 0
 * has no look-back; no wrap-around; rounds are sorted and chunked separately).
 * Keys are unit-normalised ([DT] 2.1); a zero key stays zero. Queries are not
 * normalised. Logit s_ij = (q_i . khat_j) / sqrt(d) ([DT] scaled softmax).
 * Causal: keys at a later original position are dropped.
 * Self-mask ([TT] shared-QK self-mask): the query's own key is dropped when
 * anything else is left. When nothing else is left, the query attends to
 * itself only: o = v_i and the round's logsumexp is the constant
 * LSH_ORACLE_SELF_LOGIT, which gives that round zero weight in the combine
 * step whenever another round has a real window.
 * Masked keys are excluded from the softmax (the page's multiplicative mask
 * notation is read as exclusion).
 * ------------------------------------------------------------------------- */
static void unit_key(const double* k, int64_t d, double* khat) {
  double ss = 0.0;
  for (int64_t t = 0; t < d; ++t) ss += k[t] * k[t];
  const double nrm = sqrt(ss);
  for (int64_t t = 0; t < d; ++t) khat[t] = (nrm > 0.0) ? k[t] / nrm : 0.0;
}

/* The attendable keys of the query at slot s of one round: its chunk and the
 * previous one (LOOK_AHEAD: and the next one), without the query itself,
 * (causal) later positions and (SAME_BUCKET) keys of other buckets.
 * qk_bh: [L, d] of one (b, h); pm: perm of the round; bk: the round's buckets
 * at original positions (read with SAME_BUCKET only). Writes the keys'
 * positions key[n] and logits logit[n] (n returned, at most 3m). Scratch:
 * khat [d], qhat [d]. */
static int64_t window(const lsh_oracle_config* c, const double* qk_bh, const int32_t* pm,
                      const int32_t* bk, int64_t s, double* khat, double* qhat, double* logit,
                      int64_t* key) {
  const int64_t d = c->head_dim, m = c->chunk_len, L = c->seq_len;
  const int64_t i = pm[s];
  const int64_t chunk = s / m;
  const int64_t first = (chunk > 0 ? chunk - 1 : chunk) * m;
  int64_t last = (chunk + 1) * m;
  if ((c->variant & LSH_ORACLE_LOOK_AHEAD) && last < L) last += m;
  const double* q = qk_bh + i * d;
  if (c->variant & LSH_ORACLE_NORM_QUERIES) {
    unit_key(q, d, qhat);
    q = qhat;
  }
  const double scale = 1.0 / sqrt((double)d);
  int64_t n = 0;
  for (int64_t t = first; t < last; ++t) {
    const int64_t j = pm[t];
    if (j == i) continue;                 /* self-mask */
    if (c->causal && j > i) continue;     /* causal mask on original positions */
    if ((c->variant & LSH_ORACLE_SAME_BUCKET) && bk[j] != bk[i]) continue;
    unit_key(qk_bh + j * d, d, khat);
    double dot = 0.0;
    for (int64_t u = 0; u < d; ++u) dot += q[u] * khat[u];
    logit[n] = dot * scale;
    key[n] = j;
    ++n;
  }
  return n;
}

/* DEDUP: the number of rounds in whose window key j is attendable for query
 * i (self and causal masks do not depend on the round and hold already).
 * inv_bh, bk_bh: [R, L] of one (b, h). */
static int64_t rounds_sharing(const lsh_oracle_config* c, const int32_t* inv_bh,
                              const int32_t* bk_bh, int64_t i, int64_t j) {
  const int64_t L = c->seq_len, m = c->chunk_len, R = c->n_rounds;
  int64_t n = 0;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t ci = inv_bh[r * L + i] / m, cj = inv_bh[r * L + j] / m;
    int in = cj == ci || cj == ci - 1;
    if (c->variant & LSH_ORACLE_LOOK_AHEAD) in = in || cj == ci + 1;
    if ((c->variant & LSH_ORACLE_SAME_BUCKET) && bk_bh[r * L + j] != bk_bh[r * L + i]) in = 0;
    n += in;
  }
  return n;
}

/* qk_bh, v_bh: [L, d] of one (b, h); round r; s: the query slot; pm_bh,
 * inv_bh, bk_bh: [R, L] of the (b, h) (inv_bh read with DEDUP, bk_bh with
 * SAME_BUCKET). Writes o_row [d] and returns the round's logsumexp. With
 * DEDUP each logit is lowered by log N_ij. Scratch: khat, qhat [d], logit,
 * key [3m]. */
static double attend_one(const lsh_oracle_config* c, const double* qk_bh, const double* v_bh,
                         const int32_t* pm_bh, const int32_t* inv_bh, const int32_t* bk_bh,
                         int64_t r, int64_t s, double* o_row, double* khat, double* qhat,
                         double* logit, int64_t* key) {
  const int64_t d = c->head_dim, L = c->seq_len;
  const int32_t* pm = pm_bh + r * L;
  const int64_t i = pm[s];
  const int64_t n = window(c, qk_bh, pm, bk_bh ? bk_bh + r * L : NULL, s, khat, qhat, logit,
                           key);
  if (c->variant & LSH_ORACLE_DEDUP)
    for (int64_t a = 0; a < n; ++a)
      logit[a] -= log((double)rounds_sharing(c, inv_bh, bk_bh, i, key[a]));
  if (n == 0) {
    for (int64_t u = 0; u < d; ++u) o_row[u] = v_bh[i * d + u];
    return LSH_ORACLE_SELF_LOGIT;
  }
  double mx = -INFINITY;
  for (int64_t a = 0; a < n; ++a) mx = logit[a] > mx ? logit[a] : mx;
  double sum = 0.0;
  for (int64_t a = 0; a < n; ++a) sum += exp(logit[a] - mx);
  const double lse = mx + log(sum);
  for (int64_t u = 0; u < d; ++u) o_row[u] = 0.0;
  for (int64_t a = 0; a < n; ++a) {
    const double w = exp(logit[a] - lse);
    const double* vj = v_bh + key[a] * d;
    for (int64_t u = 0; u < d; ++u) o_row[u] += w * vj[u];
  }
  return lse;
}

/* inv [nseg, L] of perm: the slot of each position, per (b, h, round) */
static int32_t* inverse_perm(const lsh_oracle_config* c, const int32_t* perm) {
  const int64_t L = c->seq_len, nseg = (int64_t)seg_count(c);
  int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(nseg * L));
  if (!inv) return NULL;
#pragma omp parallel for schedule(static)
  for (int64_t seg = 0; seg < nseg; ++seg)
    for (int64_t s = 0; s < L; ++s) inv[seg * L + perm[seg * L + s]] = (int32_t)s;
  return inv;
}

int lsh_oracle_attend(const lsh_oracle_config* c, const double* qk, const double* v,
                      const int32_t* perm, const int32_t* buckets, double* o, double* lse) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  if ((c->variant & LSH_ORACLE_SAME_BUCKET) && !buckets) return -12;
  const int64_t L = c->seq_len, d = c->head_dim, R = c->n_rounds, m = c->chunk_len;
  const int64_t nseg = (int64_t)seg_count(c);
  int32_t* inv = NULL;
  if (c->variant & LSH_ORACLE_DEDUP) {
    inv = inverse_perm(c, perm);
    if (!inv) return -8;
  }
#pragma omp parallel
  {
    double* khat = (double*)malloc(sizeof(double) * (size_t)d);
    double* qhat = (double*)malloc(sizeof(double) * (size_t)d);
    double* logit = (double*)malloc(sizeof(double) * (size_t)(3 * m));
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)(3 * m));
#pragma omp for schedule(dynamic, 1)
    for (int64_t seg = 0; seg < nseg; ++seg) {
      const int64_t bh = seg / R, r = seg % R;
      const int32_t* pm = perm + seg * L;
      for (int64_t s = 0; s < L; ++s) {
        const int64_t i = pm[s];
        /* unsort: results are stored at the original position i */
        double l = attend_one(c, qk + bh * L * d, v + bh * L * d, perm + bh * R * L,
                              inv ? inv + bh * R * L : NULL,
                              buckets ? buckets + bh * R * L : NULL, r, s,
                              o + (seg * L + i) * d, khat, qhat, logit, key);
        lse[seg * L + i] = l;
      }
    }
    free(khat);
    free(qhat);
    free(logit);
    free(key);
  }
  free(inv);
  return 0;
}

/* DEDUP, from the definition: the query at position i attends once to every
 * key that any round makes attendable for it (the union of the rounds' key
 * sets); if the union is empty it attends to itself only (out = v_i).
 * stamp [L]: scratch marking the keys already taken, with the value mark.
 * Scratch: ukey, ulogit [R * 3m] and window()'s. */
static void union_one(const lsh_oracle_config* c, const double* qk_bh, const double* v_bh,
                      const int32_t* pm_bh, const int32_t* inv_bh, const int32_t* bk_bh,
                      int64_t i, double* out_row, int64_t* stamp, int64_t mark, double* khat,
                      double* qhat, double* logit, int64_t* key, double* ulogit,
                      int64_t* ukey) {
  const int64_t d = c->head_dim, L = c->seq_len, R = c->n_rounds;
  int64_t nu = 0;
  for (int64_t r = 0; r < R; ++r) {
    const int64_t n = window(c, qk_bh, pm_bh + r * L, bk_bh ? bk_bh + r * L : NULL,
                             inv_bh[r * L + i], khat, qhat, logit, key);
    for (int64_t a = 0; a < n; ++a) {
      if (stamp[key[a]] == mark) continue;
      stamp[key[a]] = mark;
      ukey[nu] = key[a];
      ulogit[nu] = logit[a];
      ++nu;
    }
  }
  if (nu == 0) {
    for (int64_t u = 0; u < d; ++u) out_row[u] = v_bh[i * d + u];
    return;
  }
  double mx = -INFINITY;
  for (int64_t a = 0; a < nu; ++a) mx = ulogit[a] > mx ? ulogit[a] : mx;
  double sum = 0.0;
  for (int64_t a = 0; a < nu; ++a) sum += exp(ulogit[a] - mx);
  for (int64_t u = 0; u < d; ++u) out_row[u] = 0.0;
  for (int64_t a = 0; a < nu; ++a) {
    const double w = exp(ulogit[a] - mx) / sum;
    for (int64_t u = 0; u < d; ++u) out_row[u] += w * v_bh[ukey[a] * d + u];
  }
}

/* union_one for every position, or for the listed rows (rows[k] = bh * L + i;
 * all positions when rows is NULL) into out [n, d] */
static int union_rows(const lsh_oracle_config* c, const double* qk, const double* v,
                      const int32_t* perm, const int32_t* inv, const int32_t* buckets,
                      int64_t n_rows, const int64_t* rows, double* out) {
  const int64_t L = c->seq_len, d = c->head_dim, R = c->n_rounds, m = c->chunk_len;
  int bad = 0;
#pragma omp parallel
  {
    double* khat = (double*)malloc(sizeof(double) * (size_t)d);
    double* qhat = (double*)malloc(sizeof(double) * (size_t)d);
    double* logit = (double*)malloc(sizeof(double) * (size_t)(3 * m));
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)(3 * m));
    double* ulogit = (double*)malloc(sizeof(double) * (size_t)(R * 3 * m));
    int64_t* ukey = (int64_t*)malloc(sizeof(int64_t) * (size_t)(R * 3 * m));
    int64_t* stamp = (int64_t*)malloc(sizeof(int64_t) * (size_t)L);
    const int ok = khat && qhat && logit && key && ulogit && ukey && stamp;
    if (!ok) {
#pragma omp atomic write
      bad = 1;
    } else {
      for (int64_t j = 0; j < L; ++j) stamp[j] = -1;
    }
#pragma omp for schedule(dynamic, 64)
    for (int64_t k = 0; k < n_rows; ++k) {
      if (!ok) continue;
      const int64_t row = rows ? rows[k] : k;
      const int64_t bh = row / L, i = row % L;
      union_one(c, qk + bh * L * d, v + bh * L * d, perm + bh * R * L, inv + bh * R * L,
                buckets ? buckets + bh * R * L : NULL, i, out + k * d, stamp, row, khat, qhat,
                logit, key, ulogit, ukey);
    }
    free(khat);
    free(qhat);
    free(logit);
    free(key);
    free(ulogit);
    free(ukey);
    free(stamp);
  }
  return bad ? -8 : 0;
}

/* ---------------------------------------------------------------------------
 * Combination of rounds. [TT] multi-round LSH defers the details to the
 * original paper; reading taken: each round r yields o_r(i) and its logsumexp
 * lse_r(i); the rounds are combined with weights softmax over r of lse_r(i):
 *   w_r(i) = exp(lse_r(i) - M) / sum_r' exp(lse_r'(i) - M),  M = max_r lse_r(i),
 *   out(i) = sum_r w_r(i) o_r(i).
 * This equals one softmax over the multiset union of the rounds' windows
 * (a key seen in two rounds counts twice).
 * ------------------------------------------------------------------------- */
static void combine_one(int64_t R, int64_t d, const double* o_r0, int64_t o_stride,
                        const double* lse_r0, int64_t lse_stride, double* out_row) {
  double mx = -INFINITY;
  for (int64_t r = 0; r < R; ++r) mx = lse_r0[r * lse_stride] > mx ? lse_r0[r * lse_stride] : mx;
  double sum = 0.0;
  for (int64_t r = 0; r < R; ++r) sum += exp(lse_r0[r * lse_stride] - mx);
  for (int64_t u = 0; u < d; ++u) out_row[u] = 0.0;
  for (int64_t r = 0; r < R; ++r) {
    const double w = exp(lse_r0[r * lse_stride] - mx) / sum;
    const double* orow = o_r0 + r * o_stride;
    for (int64_t u = 0; u < d; ++u) out_row[u] += w * orow[u];
  }
}

int lsh_oracle_combine(const lsh_oracle_config* c, const double* o, const double* lse,
                       double* out) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  const int64_t L = c->seq_len, d = c->head_dim, R = c->n_rounds;
  const int64_t nbh = (int64_t)c->batch * c->heads;
#pragma omp parallel for schedule(static)
  for (int64_t p = 0; p < nbh * L; ++p) {
    const int64_t bh = p / L, i = p % L;
    combine_one(R, d, o + (bh * R * L + i) * d, L * d, lse + bh * R * L + i, L,
                out + p * d);
  }
  return 0;
}

int lsh_oracle_forward(const lsh_oracle_config* c, const double* qk, const double* v,
                       const double* rot, const int32_t* buckets_override, double* out,
                       double* lse, int32_t* buckets, int32_t* perm, double* margin) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  const size_t nsl = seg_count(c) * (size_t)c->seq_len;
  const size_t d = (size_t)c->head_dim;
  int32_t* bk = buckets ? buckets : (int32_t*)malloc(sizeof(int32_t) * nsl);
  int32_t* pm = perm ? perm : (int32_t*)malloc(sizeof(int32_t) * nsl);
  double* ls = lse ? lse : (double*)malloc(sizeof(double) * nsl);
  double* o = (double*)malloc(sizeof(double) * nsl * d);
  if (!bk || !pm || !ls || !o) { rc = -8; goto done; }
  if (rot || c->n_buckets == 1) {
    rc = lsh_oracle_hash(c, qk, rot, bk, margin);
    if (rc) goto done;
  }
  if (buckets_override) memcpy(bk, buckets_override, sizeof(int32_t) * nsl);
  else if (!rot && c->n_buckets > 1) { rc = -6; goto done; }
  rc = lsh_oracle_sort(c, bk, pm, NULL);
  if (rc) goto done;
  rc = lsh_oracle_attend(c, qk, v, pm, bk, o, ls);
  if (rc) goto done;
  if (c->variant & LSH_ORACLE_DEDUP) {
    int32_t* inv = inverse_perm(c, pm);
    if (!inv) { rc = -8; goto done; }
    rc = union_rows(c, qk, v, pm, inv, bk, (int64_t)c->batch * c->heads * c->seq_len, NULL,
                    out);
    free(inv);
  } else {
    rc = lsh_oracle_combine(c, o, ls, out);
  }
done:
  if (!buckets) free(bk);
  if (!perm) free(pm);
  if (!lse) free(ls);
  free(o);
  return rc;
}

/* ---------------------------------------------------------------------------
 * Backward: gradients of a loss with respect to qk and v, given dL/dout, at
 * the buckets (hence permutations) of the forward. The hash is an argmax and
 * the sort a permutation: both are piecewise constant, so no gradient flows
 * through them. The chain rule is taken through the steps above in reverse:
 *  combination (out = sum_r w_r o_r, w = softmax over rounds of lse):
 *    dL/do_r(i)   = w_r(i) dout(i)
 *    dL/dlse_r(i) = w_r(i) ((o_r(i) - out(i)) . dout(i))
 *  one round, query i with attendable keys O (softmax P_j over O):
 *    dL/dv_j     += P_j do_r(i)
 *    dL/ds_ij     = P_j (do_r(i) . v_j - sum_k P_k do_r(i) . v_k) + P_j dlse_r(i)
 *    with s_ij = (q_i . khat_j) / sqrt(d), q_i = qk_i, khat_j = qk_j / |qk_j|:
 *    dL/dq_i     += dL/ds_ij khat_j / sqrt(d),   dL/dkhat_j += dL/ds_ij q_i / sqrt(d)
 *  a query that could attend only to itself has o_r(i) = v_i:
 *    dL/dv_i     += do_r(i)   (its logsumexp is a constant)
 *  key normalisation (khat = k / |k|, khat := 0 for k = 0):
 *    dL/dk_j      = (dkhat_j - khat_j (khat_j . dkhat_j)) / |k_j|
 *  shared QK: dL/dqk_j = dL/dq_j + dL/dk_j.
 * The variant readings change only which keys are attendable and the logits,
 * exactly as in the forward (window(), and with DEDUP s_ij lowered by the
 * constant log N_ij), except NORM_QUERIES, where s_ij uses the unit query
 * qhat_i = q_i / |q_i|: then dL/dqhat_i += dL/ds_ij khat_j / sqrt(d), the key
 * term uses qhat_i, and qhat_i goes through the same normalisation Jacobian as
 * khat_i (they are the same unit vector of qk_i).
 * perm: every round's permutation [B, H, R, L]; buckets [B, H, R, L] (read
 * with SAME_BUCKET, else may be NULL); dout, dqk, dv: [B, H, L, d].
 * ------------------------------------------------------------------------- */
int lsh_oracle_backward(const lsh_oracle_config* c, const double* qk, const double* v,
                        const int32_t* perm, const int32_t* buckets, const double* dout,
                        double* dqk, double* dv) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  if ((c->variant & LSH_ORACLE_SAME_BUCKET) && !buckets) return -12;
  const int64_t L = c->seq_len, d = c->head_dim, R = c->n_rounds, m = c->chunk_len;
  const int64_t nbh = (int64_t)c->batch * c->heads;
  const size_t nsl = seg_count(c) * (size_t)L;
  double* o = (double*)malloc(sizeof(double) * nsl * (size_t)d);
  double* lse = (double*)malloc(sizeof(double) * nsl);
  double* out = (double*)malloc(sizeof(double) * (size_t)(nbh * L * d));
  double* dkhat = (double*)calloc((size_t)(nbh * L * d), sizeof(double));
  int32_t* inv = (c->variant & LSH_ORACLE_DEDUP) ? inverse_perm(c, perm) : NULL;
  if (!o || !lse || !out || !dkhat || ((c->variant & LSH_ORACLE_DEDUP) && !inv)) {
    rc = -8;
    goto done;
  }
  rc = lsh_oracle_attend(c, qk, v, perm, buckets, o, lse);
  if (rc) goto done;
  rc = lsh_oracle_combine(c, o, lse, out);
  if (rc) goto done;
  for (int64_t x = 0; x < nbh * L * d; ++x) { dqk[x] = 0.0; dv[x] = 0.0; }
  /* one (b, h) per thread: every write of a (b, h) stays in its own rows */
#pragma omp parallel
  {
    double* khat = (double*)malloc(sizeof(double) * (size_t)d);
    double* qhat = (double*)malloc(sizeof(double) * (size_t)d);
    double* logit = (double*)malloc(sizeof(double) * (size_t)(3 * m));
    double* pj = (double*)malloc(sizeof(double) * (size_t)(3 * m));
    double* dp = (double*)malloc(sizeof(double) * (size_t)(3 * m));
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)(3 * m));
    double* dor = (double*)malloc(sizeof(double) * (size_t)d);
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < nbh; ++bh) {
      const double* qk_bh = qk + bh * L * d;
      const double* v_bh = v + bh * L * d;
      for (int64_t r = 0; r < R; ++r) {
        const int64_t seg = bh * R + r;
        const int32_t* pm = perm + seg * L;
        for (int64_t s = 0; s < L; ++s) {
          const int64_t i = pm[s];
          /* combination backward for (round r, position i) */
          double mx = -INFINITY;
          for (int64_t rr = 0; rr < R; ++rr) {
            const double l = lse[(bh * R + rr) * L + i];
            mx = l > mx ? l : mx;
          }
          double sum = 0.0;
          for (int64_t rr = 0; rr < R; ++rr) sum += exp(lse[(bh * R + rr) * L + i] - mx);
          const double w = exp(lse[seg * L + i] - mx) / sum;
          const double* orow = o + (seg * L + i) * d;
          const double* outrow = out + (bh * L + i) * d;
          const double* drow = dout + (bh * L + i) * d;
          double g = 0.0;
          for (int64_t u = 0; u < d; ++u) {
            dor[u] = w * drow[u];
            g += (orow[u] - outrow[u]) * drow[u];
          }
          const double dlse = w * g;
          /* the round's window and logits, as in the forward (with
           * NORM_QUERIES, window() leaves the unit query in qhat) */
          const int64_t n = window(c, qk_bh, pm, buckets ? buckets + seg * L : NULL, s, khat,
                                   qhat, logit, key);
          if (c->variant & LSH_ORACLE_DEDUP)
            for (int64_t a = 0; a < n; ++a)
              logit[a] -= log((double)rounds_sharing(c, inv + bh * R * L,
                                                     buckets ? buckets + bh * R * L : NULL, i,
                                                     key[a]));
          const int nq = (c->variant & LSH_ORACLE_NORM_QUERIES) != 0;
          const double* q = nq ? qhat : qk_bh + i * d;
          const double scale = 1.0 / sqrt((double)d);
          if (n == 0) {
            for (int64_t u = 0; u < d; ++u) dv[(bh * L + i) * d + u] += dor[u];
            continue;
          }
          const double l = lse[seg * L + i];
          double dsum = 0.0;
          for (int64_t a = 0; a < n; ++a) {
            pj[a] = exp(logit[a] - l);
            double t = 0.0;
            for (int64_t u = 0; u < d; ++u) t += dor[u] * v_bh[key[a] * d + u];
            dp[a] = t;
            dsum += pj[a] * t;
          }
          for (int64_t a = 0; a < n; ++a) {
            const int64_t j = key[a];
            const double ds = pj[a] * (dp[a] - dsum) + pj[a] * dlse;
            unit_key(qk_bh + j * d, d, khat);
            /* the query's own gradient: with NORM_QUERIES it is taken with
             * respect to the unit query, which shares the key's Jacobian */
            double* dqi = nq ? dkhat + (bh * L + i) * d : dqk + (bh * L + i) * d;
            for (int64_t u = 0; u < d; ++u) {
              dv[(bh * L + j) * d + u] += pj[a] * dor[u];
              dqi[u] += ds * khat[u] * scale;
              dkhat[(bh * L + j) * d + u] += ds * q[u] * scale;
            }
          }
        }
      }
      /* normalisation of the keys (and of the queries with NORM_QUERIES):
       * x / |x| has the Jacobian (I - xhat xhat^T) / |x| */
      for (int64_t j = 0; j < L; ++j) {
        const double* k = qk_bh + j * d;
        double ss = 0.0;
        for (int64_t u = 0; u < d; ++u) ss += k[u] * k[u];
        const double nrm = sqrt(ss);
        if (nrm == 0.0) continue;
        const double* dk = dkhat + (bh * L + j) * d;
        double proj = 0.0;
        for (int64_t u = 0; u < d; ++u) proj += (k[u] / nrm) * dk[u];
        for (int64_t u = 0; u < d; ++u)
          dqk[(bh * L + j) * d + u] += (dk[u] - (k[u] / nrm) * proj) / nrm;
      }
    }
    free(khat);
    free(qhat);
    free(logit);
    free(pj);
    free(dp);
    free(key);
    free(dor);
  }
done:
  free(o);
  free(lse);
  free(out);
  free(dkhat);
  free(inv);
  return rc;
}

/* ---------------------------------------------------------------------------
 * Magnitudes of the backward's terms, for error bounds on a finite-precision
 * backward (test infrastructure: the tolerance of a GPU backward is a unit
 * roundoff times these sums). Same traversal as lsh_oracle_backward, with
 * every term replaced by an upper bound of its absolute value:
 *   A_ij   = w_r(i) P_ij (|dout_i . v_j| + |dout_i . out_i| + 2 E_i),
 *            E_i = sum over rounds r' of w_r'(i) sum_j' P_ij' |dout_i . v_j'|,
 *            which bounds |dS_ij| and also scales the error of dS_ij that
 *            comes from an inexact dout_i . out_i;
 *   mdv[j] += w_r(i) P_ij |dout_i|            (elementwise; self-only rounds:
 *                                              w_r(i) |dout_i| at i);
 *   mdq[i] += A_ij |khat_j| / sqrt(d),  mdk[j] += A_ij |q_i| / sqrt(d);
 *   mdqk   = mdq + (|mdk| + |khat| (|khat| . mdk)) / |k|   (the normalisation's
 *            Jacobian with every term taken in absolute value).
 * So |dv| <= mdv and |dqk| <= mdqk elementwise (triangle inequality), with
 * equality for dv when every dout and v entry is non-negative. The variant
 * readings change the windows and logits as in the forward; with
 * NORM_QUERIES q_i is the unit query and its term goes into mdk[i]. */
int lsh_oracle_backward_magnitudes(const lsh_oracle_config* c, const double* qk,
                                   const double* v, const int32_t* perm, const int32_t* buckets,
                                   const double* dout, double* mdqk, double* mdv) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  if ((c->variant & LSH_ORACLE_SAME_BUCKET) && !buckets) return -12;
  const int64_t L = c->seq_len, d = c->head_dim, R = c->n_rounds, m = c->chunk_len;
  const int64_t nbh = (int64_t)c->batch * c->heads;
  const size_t nsl = seg_count(c) * (size_t)L;
  double* o = (double*)malloc(sizeof(double) * nsl * (size_t)d);
  double* lse = (double*)malloc(sizeof(double) * nsl);
  double* out = (double*)malloc(sizeof(double) * (size_t)(nbh * L * d));
  double* mdk = (double*)calloc((size_t)(nbh * L * d), sizeof(double));
  double* eq = (double*)calloc((size_t)(nbh * L), sizeof(double));
  int32_t* inv = (c->variant & LSH_ORACLE_DEDUP) ? inverse_perm(c, perm) : NULL;
  if (!o || !lse || !out || !mdk || !eq || ((c->variant & LSH_ORACLE_DEDUP) && !inv)) {
    rc = -8;
    goto done;
  }
  rc = lsh_oracle_attend(c, qk, v, perm, buckets, o, lse);
  if (rc) goto done;
  rc = lsh_oracle_combine(c, o, lse, out);
  if (rc) goto done;
  for (int64_t x = 0; x < nbh * L * d; ++x) { mdqk[x] = 0.0; mdv[x] = 0.0; }
#pragma omp parallel
  {
    double* khat = (double*)malloc(sizeof(double) * (size_t)d);
    double* qhat = (double*)malloc(sizeof(double) * (size_t)d);
    double* logit = (double*)malloc(sizeof(double) * (size_t)(3 * m));
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)(3 * m));
#pragma omp for schedule(dynamic, 1)
    for (int64_t bh = 0; bh < nbh; ++bh) {
      const double* qk_bh = qk + bh * L * d;
      const double* v_bh = v + bh * L * d;
      /* two passes over the rounds: E_i first, then the sums */
      for (int pass = 0; pass < 2; ++pass) {
        for (int64_t r = 0; r < R; ++r) {
          const int64_t seg = bh * R + r;
          const int32_t* pm = perm + seg * L;
          for (int64_t s = 0; s < L; ++s) {
            const int64_t i = pm[s];
            double mx = -INFINITY;
            for (int64_t rr = 0; rr < R; ++rr) {
              const double l = lse[(bh * R + rr) * L + i];
              mx = l > mx ? l : mx;
            }
            double sum = 0.0;
            for (int64_t rr = 0; rr < R; ++rr) sum += exp(lse[(bh * R + rr) * L + i] - mx);
            const double w = exp(lse[seg * L + i] - mx) / sum;
            const double* drow = dout + (bh * L + i) * d;
            const int64_t n = window(c, qk_bh, pm, buckets ? buckets + seg * L : NULL, s, khat,
                                     qhat, logit, key);
            if (c->variant & LSH_ORACLE_DEDUP)
              for (int64_t a = 0; a < n; ++a)
                logit[a] -= log((double)rounds_sharing(c, inv + bh * R * L,
                                                       buckets ? buckets + bh * R * L : NULL, i,
                                                       key[a]));
            if (n == 0) {
              if (pass == 1)
                for (int64_t u = 0; u < d; ++u) mdv[(bh * L + i) * d + u] += w * fabs(drow[u]);
              continue;
            }
            const double l = lse[seg * L + i];
            const double* outrow = out + (bh * L + i) * d;
            double dq_out = 0.0;
            for (int64_t u = 0; u < d; ++u) dq_out += drow[u] * outrow[u];
            const int nq = (c->variant & LSH_ORACLE_NORM_QUERIES) != 0;
            const double* q = nq ? qhat : qk_bh + i * d;
            const double scale = 1.0 / sqrt((double)d);
            for (int64_t a = 0; a < n; ++a) {
              const int64_t j = key[a];
              const double wp = w * exp(logit[a] - l);
              double dpv = 0.0;
              for (int64_t u = 0; u < d; ++u) dpv += drow[u] * v_bh[j * d + u];
              if (pass == 0) {
                eq[bh * L + i] += wp * fabs(dpv);
                continue;
              }
              const double A = wp * (fabs(dpv) + fabs(dq_out) + 2.0 * eq[bh * L + i]);
              unit_key(qk_bh + j * d, d, khat);
              double* mqi = nq ? mdk + (bh * L + i) * d : mdqk + (bh * L + i) * d;
              for (int64_t u = 0; u < d; ++u) {
                mdv[(bh * L + j) * d + u] += wp * fabs(drow[u]);
                mqi[u] += A * fabs(khat[u]) * scale;
                mdk[(bh * L + j) * d + u] += A * fabs(q[u]) * scale;
              }
            }
          }
        }
      }
      for (int64_t j = 0; j < L; ++j) {
        const double* k = qk_bh + j * d;
        double ss = 0.0;
        for (int64_t u = 0; u < d; ++u) ss += k[u] * k[u];
        const double nrm = sqrt(ss);
        if (nrm == 0.0) continue;
        const double* mk = mdk + (bh * L + j) * d;
        double proj = 0.0;
        for (int64_t u = 0; u < d; ++u) proj += fabs(k[u] / nrm) * mk[u];
        for (int64_t u = 0; u < d; ++u)
          mdqk[(bh * L + j) * d + u] += (mk[u] + fabs(k[u] / nrm) * proj) / nrm;
      }
    }
    free(khat);
    free(qhat);
    free(logit);
    free(key);
  }
done:
  free(o);
  free(lse);
  free(out);
  free(mdk);
  free(eq);
  free(inv);
  return rc;
}

int lsh_oracle_attend_rows(const lsh_oracle_config* c, const double* qk, const double* v,
                           const int32_t* perm, const int32_t* buckets, int64_t n_rows,
                           const int64_t* rows, double* out_rows, double* lse_rows) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  if ((c->variant & LSH_ORACLE_SAME_BUCKET) && !buckets) return -12;
  const int64_t L = c->seq_len, d = c->head_dim, R = c->n_rounds, m = c->chunk_len;
  const int64_t nbh = (int64_t)c->batch * c->heads;
  for (int64_t k = 0; k < n_rows; ++k)
    if (rows[k] < 0 || rows[k] >= nbh * L) return -9;
  int32_t* inv = inverse_perm(c, perm);
  if (!inv) return -8;
#pragma omp parallel
  {
    double* khat = (double*)malloc(sizeof(double) * (size_t)d);
    double* qhat = (double*)malloc(sizeof(double) * (size_t)d);
    double* logit = (double*)malloc(sizeof(double) * (size_t)(3 * m));
    int64_t* key = (int64_t*)malloc(sizeof(int64_t) * (size_t)(3 * m));
    double* o = (double*)malloc(sizeof(double) * (size_t)(R * d));
    double* l = (double*)malloc(sizeof(double) * (size_t)R);
#pragma omp for schedule(dynamic, 16)
    for (int64_t k = 0; k < n_rows; ++k) {
      const int64_t bh = rows[k] / L, i = rows[k] % L;
      for (int64_t r = 0; r < R; ++r) {
        const int64_t seg = bh * R + r;
        const int64_t s = inv[seg * L + i];
        l[r] = attend_one(c, qk + bh * L * d, v + bh * L * d, perm + bh * R * L,
                          inv + bh * R * L, buckets ? buckets + bh * R * L : NULL, r, s,
                          o + r * d, khat, qhat, logit, key);
        if (lse_rows) lse_rows[k * R + r] = l[r];
      }
      if (!(c->variant & LSH_ORACLE_DEDUP)) combine_one(R, d, o, d, l, 1, out_rows + k * d);
    }
    free(khat);
    free(qhat);
    free(logit);
    free(key);
    free(o);
    free(l);
  }
  if (c->variant & LSH_ORACLE_DEDUP)
    rc = union_rows(c, qk, v, perm, inv, buckets, n_rows, rows, out_rows);
  free(inv);
  return rc;
}

/* ---------------------------------------------------------------------------
 * Projections ([TT] shared-QK section): qk and v of every head from the layer
 * input, one dot product per output element, summed over k in order.
 * ------------------------------------------------------------------------- */
int lsh_oracle_project(const lsh_oracle_config* c, int64_t model_dim, const double* x,
                       const double* w_qk, const double* w_v, double* qk, double* v) {
  int rc = lsh_oracle_check(c);
  if (rc) return rc;
  if (model_dim < 1) return -13;
  const int64_t B = c->batch, H = c->heads, L = c->seq_len, d = c->head_dim;
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t i = 0; i < L; ++i) {
        const double* xr = x + (b * L + i) * model_dim;
        for (int64_t e = 0; e < d; ++e) {
          const double* wq = w_qk + (h * d + e) * model_dim;
          const double* wv = w_v + (h * d + e) * model_dim;
          double sq = 0.0, sv = 0.0;
          for (int64_t k = 0; k < model_dim; ++k) {
            sq += xr[k] * wq[k];
            sv += xr[k] * wv[k];
          }
          qk[((b * H + h) * L + i) * d + e] = sq;
          v[((b * H + h) * L + i) * d + e] = sv;
        }
      }
  return 0;
}

/* ---------------------------------------------------------------------------
 * Chunked feed-forward, [DT] section 2.3: the feed-forward is applied to one
 * chunk of rows at a time and the chunk outputs are concatenated; d_ff is
 * usually four times the model dimension. [TT] "FF layer chunking" splits
 * the second half of the reversible block, y2 = x2 + FF(y1), the same way.
 * Readings where the pages are silent: FF is the plain two-layer feed-forward
 * with biases and a ReLU between the layers (no normalisation inside), and
 * the residual x2 is added to its output when given.
 * Each chunk holds its own hidden activations [chunk_rows, d_ff] (the memory
 * the chunking bounds); every row is computed the same way in any chunk.
 */
int lsh_oracle_ffn(int64_t rows, int64_t d_model, int64_t d_ff, int64_t chunk_rows,
                   const double* y1, const double* w1, const double* b1, const double* w2,
                   const double* b2, const double* x2, double* y2, double* hidden) {
  if (rows < 0 || d_model < 1 || d_ff < 1 || chunk_rows < 1) return -13;
  if (rows == 0) return 0;
  const int64_t cr = chunk_rows < rows ? chunk_rows : rows;
  double* h = (double*)malloc(sizeof(double) * (size_t)(cr * d_ff));
  if (!h) return -12;
  for (int64_t c0 = 0; c0 < rows; c0 += cr) {
    const int64_t n = (rows - c0 < cr) ? rows - c0 : cr;  /* rows in this chunk */
    /* first layer and ReLU */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      const double* yr = y1 + (c0 + r) * d_model;
      for (int64_t j = 0; j < d_ff; ++j) {
        const double* wj = w1 + j * d_model;
        double s = 0.0;
        for (int64_t k = 0; k < d_model; ++k) s += yr[k] * wj[k];
        s += b1[j];
        h[r * d_ff + j] = s > 0.0 ? s : 0.0;
      }
    }
    /* second layer, bias, residual */
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
      const double* hr = h + r * d_ff;
      for (int64_t e = 0; e < d_model; ++e) {
        const double* we = w2 + e * d_ff;
        double s = 0.0;
        for (int64_t j = 0; j < d_ff; ++j) s += hr[j] * we[j];
        s += b2[e];
        if (x2) s += x2[(c0 + r) * d_model + e];
        y2[(c0 + r) * d_model + e] = s;
      }
    }
    if (hidden) memcpy(hidden + c0 * d_ff, h, sizeof(double) * (size_t)(n * d_ff));
  }
  free(h);
  return 0;
}
