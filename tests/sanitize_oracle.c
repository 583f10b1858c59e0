/* Runs every entry point of oracle/ra_oracle.c once on small seeded inputs,
 * for a build under AddressSanitizer and UndefinedBehaviorSanitizer
 * (tests/test_sanitize.py).  Checks only that each call returns 0 and gives
 * finite results; the values are pinned elsewhere.  Prints "ok". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int orc_attention(const double *q, const double *k, const double *v, int64_t B, int64_t q_rows, int64_t kv_rows,
                  int64_t nq, int64_t nkv, int64_t hq, int64_t hkv, int64_t d, int64_t q_off, int64_t kv_off,
                  int causal, double scale, const int64_t *rows, int64_t nrows, double *o, double *lse,
                  int nthreads);
int orc_block_partial(const double *q, const double *k, const double *v, int64_t B, int64_t q_rows,
                      int64_t kv_rows, int64_t nq, int64_t nkv, int64_t hq, int64_t hkv, int64_t d, int64_t q_off,
                      int64_t kv_off, int causal, double scale, const int64_t *rows, int64_t nrows, double *m,
                      double *l, double *o, int nthreads);
void orc_merge(int64_t nrows, int64_t d, const double *ma, const double *la, const double *oa, const double *mb,
               const double *lb, const double *ob, double *m, double *l, double *o);
void orc_finalize(int64_t nrows, int64_t d, const double *m, const double *l, const double *o, double *out,
                  double *lse);
int64_t orc_ring_block(int64_t P, int64_t rank, int64_t s);
int orc_rank_share(const double *q, const double *k, const double *v, int64_t B, int64_t N, int64_t P,
                   int64_t rank, int64_t hq, int64_t hkv, int64_t d, int causal, double scale, const int64_t *rows,
                   int64_t nrows, double *out, double *lse, int nthreads);
int orc_rank_share_padded(const double *q, const double *k, const double *v, int64_t B, int64_t N, int64_t P,
                          int64_t rank, int64_t hq, int64_t hkv, int64_t d, int causal, double scale,
                          int64_t n_valid, const int64_t *rows, int64_t nrows, double *out, double *lse,
                          int nthreads);
int orc_rank_share_zigzag(const double *q, const double *k, const double *v, int64_t B, int64_t N, int64_t P,
                          int64_t rank, int64_t hq, int64_t hkv, int64_t d, int causal, double scale,
                          const int64_t *rows, int64_t nrows, double *out, double *lse, int nthreads);
int orc_classify(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal);
int64_t orc_visible_pairs(int64_t q_off, int64_t nq, int64_t kv_off, int64_t nkv, int causal);
double orc_share_flops(int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t d, int causal);
double orc_share_flops_zigzag(int64_t B, int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t d, int causal);
int orc_rank_share_bwd(const double *q, const double *k, const double *v, const double *dout, int64_t B, int64_t N,
                       int64_t P, int64_t rank, int64_t hq, int64_t hkv, int64_t d, int causal, double scale,
                       const int64_t *qrows, int64_t nqrows, const int64_t *krows, int64_t nkrows, double *dq,
                       double *dk, double *dv, int nthreads);
int orc_rank_share_padded_bwd(const double *q, const double *k, const double *v, const double *dout, int64_t B,
                              int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t hkv, int64_t d, int causal,
                              double scale, int64_t n_valid, const int64_t *qrows, int64_t nqrows,
                              const int64_t *krows, int64_t nkrows, double *dq, double *dk, double *dv,
                              int nthreads);
int orc_rank_share_zigzag_bwd(const double *q, const double *k, const double *v, const double *dout, int64_t B,
                              int64_t N, int64_t P, int64_t rank, int64_t hq, int64_t hkv, int64_t d, int causal,
                              double scale, const int64_t *qrows, int64_t nqrows, const int64_t *krows,
                              int64_t nkrows, double *dq, double *dk, double *dv, int nthreads);

static uint64_t g_state = 12345;
static double rnd(void) { /* uniform in [-1, 1) from a 64-bit LCG */
  g_state = g_state * 6364136223846793005ULL + 1442695040888963407ULL;
  return (double)(g_state >> 11) / 9007199254740992.0 * 2.0 - 1.0;
}
static double *arr(int64_t n) {
  double *a = malloc((size_t)n * sizeof(double));
  for (int64_t i = 0; i < n; ++i) a[i] = rnd();
  return a;
}
/* (b, h, i) rows of every local row */
static int64_t *rows_all(int64_t B, int64_t H, int64_t n) {
  int64_t *r = malloc((size_t)(B * H * n * 3) * sizeof(int64_t)), t = 0;
  for (int64_t b = 0; b < B; ++b)
    for (int64_t h = 0; h < H; ++h)
      for (int64_t i = 0; i < n; ++i) r[3 * t] = b, r[3 * t + 1] = h, r[3 * t + 2] = i, ++t;
  return r;
}
static int finite_all(const double *a, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}
#define CHECK(cond, what)                     \
  do {                                        \
    if (!(cond)) {                            \
      printf("failed: %s\n", what);           \
      return 1;                               \
    }                                         \
  } while (0)

int main(void) {
  const int64_t B = 2, N = 24, P = 3, hq = 4, hkv = 2, d = 8, nb = N / P, nz = N / P;
  const double scale = 1.0 / sqrt((double)d);
  double *qf = arr(B * N * hq * d), *k = arr(B * N * hkv * d), *v = arr(B * N * hkv * d);
  double *ql = arr(B * nb * hq * d), *dout = arr(B * nb * hq * d);
  int64_t *rows = rows_all(B, hq, nb), *qrows = rows_all(B, hq, nb), *krows = rows_all(B, hkv, N);
  const int64_t nr = B * hq * nb, nk = B * hkv * N;
  double *o = malloc(nr * d * sizeof(double)), *lse = malloc(nr * sizeof(double));
  double *m = malloc(nr * sizeof(double)), *l = malloc(nr * sizeof(double)), *ob = malloc(nr * d * sizeof(double));
  double *m2 = malloc(nr * sizeof(double)), *l2 = malloc(nr * sizeof(double)), *o2 = malloc(nr * d * sizeof(double));
  double *dq = malloc(nr * d * sizeof(double)), *dk = malloc(nk * d * sizeof(double)),
         *dv = malloc(nk * d * sizeof(double));
  for (int causal = 0; causal < 2; ++causal) {
    CHECK(orc_attention(qf, k, v, B, N, N, N, N, hq, hkv, d, 0, 0, causal, scale, rows, nr, o, lse, 3) == 0,
          "attention");
    CHECK(finite_all(o, nr * d) && finite_all(lse, nr), "attention finite");
    CHECK(orc_block_partial(ql, k, v, B, nb, N, nb, nb, hq, hkv, d, 2 * nb, nb, causal, scale, rows, nr, m, l, ob,
                            2) == 0,
          "block_partial");
    CHECK(orc_block_partial(ql, k, v, B, nb, N, nb, nb, hq, hkv, d, 2 * nb, 2 * nb, causal, scale, rows, nr, m2,
                            l2, o2, 2) == 0,
          "block_partial 2");
    orc_merge(nr, d, m, l, ob, m2, l2, o2, m, l, ob);
    orc_finalize(nr, d, m, l, ob, o, lse);
    CHECK(finite_all(o, nr * d) && finite_all(lse, nr), "merge + finalize finite");
    for (int64_t r = 0; r < P; ++r) {
      CHECK(orc_rank_share(ql, k, v, B, N, P, r, hq, hkv, d, causal, scale, rows, nr, o, lse, 4) == 0, "share");
      CHECK(finite_all(o, nr * d), "share finite");
      CHECK(orc_rank_share_padded(ql, k, v, B, N, P, r, hq, hkv, d, causal, scale, N - 5, rows, nr, o, lse, 4) == 0,
            "padded share");
      CHECK(orc_rank_share_zigzag(ql, k, v, B, N, P, r, hq, hkv, d, causal, scale, rows, nr, o, lse, 4) == 0,
            "zigzag share");
      CHECK(orc_rank_share_bwd(ql, k, v, dout, B, N, P, r, hq, hkv, d, causal, scale, qrows, nr, krows, nk, dq, dk,
                               dv, 3) == 0,
            "share backward");
      CHECK(finite_all(dq, nr * d) && finite_all(dk, nk * d) && finite_all(dv, nk * d), "backward finite");
      CHECK(orc_rank_share_padded_bwd(ql, k, v, dout, B, N, P, r, hq, hkv, d, causal, scale, N - 5, qrows, nr, krows,
                                      nk, dq, dk, dv, 3) == 0,
            "padded backward");
      CHECK(orc_rank_share_zigzag_bwd(ql, k, v, dout, B, N, P, r, hq, hkv, d, causal, scale, qrows, nr, krows, nk,
                                      dq, dk, dv, 3) == 0,
            "zigzag backward");
      CHECK(orc_share_flops(B, N, P, r, hq, d, causal) > 0 && orc_share_flops_zigzag(B, N, P, r, hq, d, causal) > 0,
            "flops");
    }
  }
  int64_t pairs = 0;
  for (int64_t a = 0; a < 12; ++a)
    for (int64_t b = 0; b < 12; ++b) {
      pairs += orc_visible_pairs(a, 5, b, 7, 1);
      CHECK(orc_classify(a, 5, b, 7, 1) >= 0 && orc_ring_block(5, a % 5, b) >= 0, "classes");
    }
  CHECK(pairs > 0 && nz == nb, "pairs");
  free(qf); free(k); free(v); free(ql); free(dout); free(rows); free(qrows); free(krows); free(o); free(lse);
  free(m); free(l); free(ob); free(m2); free(l2); free(o2); free(dq); free(dk); free(dv);
  printf("ok\n");
  return 0;
}
