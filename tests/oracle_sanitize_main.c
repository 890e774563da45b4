/* Drives every entry point of the fp64 oracle (oracle/lsh_oracle.c) on small
 * seeded inputs so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer checks its index arithmetic: windows at chunk 0
 * and the last chunk, look-ahead past the end, ragged feed-forward chunks, the
 * de-duplication counts over rounds, zero rows, one bucket, odd shapes. It
 * checks no values (the Python pins do that); a sanitizer report or a
 * non-zero status from the oracle fails it. Built and run by
 * tests/test_oracle_sanitize.py. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include "lsh_oracle.h"

static uint64_t state = 88172645463325252ull;
static double uniform(void) {  /* xorshift64, in [-1, 1) */
  state ^= state << 13;
  state ^= state >> 7;
  state ^= state << 17;
  return (double)(state >> 11) / (double)(1ull << 52) - 1.0;
}
static double* fill(size_t n) {
  double* p = (double*)malloc(sizeof(double) * (n ? n : 1));
  for (size_t i = 0; i < n; ++i) p[i] = uniform();
  return p;
}

#define CHECK(call)                                              \
  do {                                                           \
    int rc_ = (call);                                            \
    if (rc_ != 0) {                                              \
      fprintf(stderr, "%s returned %d (line %d)\n", #call, rc_, __LINE__); \
      return 1;                                                  \
    }                                                            \
  } while (0)

static int one_case(int B, int H, int L, int d, int nb, int R, int m, int causal, int variant) {
  lsh_oracle_config c = {B, H, L, d, nb, R, m, causal, variant};
  const size_t tok = (size_t)B * H * L, rows = tok * R;
  double* qk = fill(tok * d);
  double* v = fill(tok * d);
  double* rot = nb > 1 ? fill((size_t)R * d * (nb / 2)) : NULL;
  double* dout = fill(tok * d);
  for (int i = 0; i < d; ++i) qk[i] = 0.0; /* a zero row */
  int32_t* bk = (int32_t*)malloc(sizeof(int32_t) * rows);
  int32_t* pm = (int32_t*)malloc(sizeof(int32_t) * rows);
  int32_t* iv = (int32_t*)malloc(sizeof(int32_t) * rows);
  double* mg = (double*)malloc(sizeof(double) * rows);
  double* o = (double*)malloc(sizeof(double) * rows * d);
  double* lse = (double*)malloc(sizeof(double) * rows);
  double* out = (double*)malloc(sizeof(double) * tok * d);
  double* dqk = (double*)malloc(sizeof(double) * tok * d);
  double* dv = (double*)malloc(sizeof(double) * tok * d);
  CHECK(lsh_oracle_hash(&c, qk, rot, bk, mg));
  CHECK(lsh_oracle_sort(&c, bk, pm, iv));
  CHECK(lsh_oracle_attend(&c, qk, v, pm, bk, o, lse));
  if (!(variant & LSH_ORACLE_DEDUP)) CHECK(lsh_oracle_combine(&c, o, lse, out));
  CHECK(lsh_oracle_forward(&c, qk, v, rot, NULL, out, lse, bk, pm, mg));
  CHECK(lsh_oracle_forward(&c, qk, v, rot, bk, out, NULL, NULL, NULL, NULL));
  int64_t sample[4] = {0, L - 1, (int64_t)tok - 1, (int64_t)tok / 2};
  double* orow = (double*)malloc(sizeof(double) * 4 * d);
  double* lrow = (double*)malloc(sizeof(double) * 4 * R);
  CHECK(lsh_oracle_attend_rows(&c, qk, v, pm, bk, 4, sample, orow, lrow));
  CHECK(lsh_oracle_backward(&c, qk, v, pm, bk, dout, dqk, dv));
  {
    double* mq = (double*)malloc(sizeof(double) * tok * d);
    double* mv = (double*)malloc(sizeof(double) * tok * d);
    CHECK(lsh_oracle_backward_magnitudes(&c, qk, v, pm, bk, dout, mq, mv));
    free(mq);
    free(mv);
  }
  const int64_t md = 24;
  double* x = fill((size_t)B * L * md);
  double* wq = fill((size_t)H * d * md);
  double* wv = fill((size_t)H * d * md);
  CHECK(lsh_oracle_project(&c, md, x, wq, wv, dqk, dv));
  free(x); free(wq); free(wv); free(orow); free(lrow);
  free(qk); free(v); free(rot); free(dout); free(bk); free(pm); free(iv); free(mg);
  free(o); free(lse); free(out); free(dqk); free(dv);
  return 0;
}

static int ffn_case(int64_t rows, int64_t dm, int64_t dff, int64_t chunk, int residual) {
  double* y1 = fill((size_t)rows * dm);
  double* w1 = fill((size_t)dff * dm);
  double* b1 = fill((size_t)dff);
  double* w2 = fill((size_t)dm * dff);
  double* b2 = fill((size_t)dm);
  double* x2 = residual ? fill((size_t)rows * dm) : NULL;
  double* y2 = (double*)malloc(sizeof(double) * (size_t)(rows ? rows : 1) * dm);
  double* hid = (double*)malloc(sizeof(double) * (size_t)(rows ? rows : 1) * dff);
  CHECK(lsh_oracle_ffn(rows, dm, dff, chunk, y1, w1, b1, w2, b2, x2, y2, hid));
  free(y1); free(w1); free(b1); free(w2); free(b2); free(x2); free(y2); free(hid);
  return 0;
}

int main(void) {
  const int variants[] = {0, LSH_ORACLE_LOOK_AHEAD, LSH_ORACLE_SAME_BUCKET,
                          LSH_ORACLE_NORM_QUERIES, LSH_ORACLE_DEDUP, 15};
  for (int vi = 0; vi < 6; ++vi)
    for (int causal = 0; causal < 2; ++causal) {
      if (one_case(2, 2, 48, 8, 6, 3, 8, causal, variants[vi])) return 1;   /* 6 chunks */
      if (one_case(1, 1, 16, 4, 4, 2, 16, causal, variants[vi])) return 1;  /* one chunk */
      if (one_case(1, 2, 12, 3, 1, 2, 4, causal, variants[vi])) return 1;   /* one bucket */
      if (one_case(1, 1, 10, 5, 2, 5, 1, causal, variants[vi])) return 1;   /* chunk of 1 */
    }
  if (ffn_case(37, 8, 16, 10, 1)) return 1;  /* ragged last chunk */
  if (ffn_case(5, 4, 8, 5, 0)) return 1;     /* one chunk, no residual */
  if (ffn_case(0, 4, 8, 3, 1)) return 1;     /* no rows */
  printf("oracle sanitizer drive ok\n");
  return 0;
}
