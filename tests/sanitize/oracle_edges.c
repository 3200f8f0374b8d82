/*
 * Edge cases of the fp64 oracle, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer (see tests/test_sanitizers.py).  Every buffer is
 * allocated at exactly the size the oracle's layout needs, so a read or write
 * past it stops the run.  Checks are structural (return codes, finiteness,
 * rows that see no key): the numerical pins of the oracle live in the Python
 * tests.  Exit status 0 = every case behaved.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int oracle_fwd_rows(const double *q, const double *k, const double *v, long B, long H, long N,
                    long d, double scale, int causal, const long *rows, long nrows, double *o_rows,
                    double *lse_rows, int nthreads);
int oracle_fwd(const double *q, const double *k, const double *v, long B, long H, long N, long d,
               double scale, int causal, double *o, double *lse, int nthreads);
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
int oracle_dropout_mask(long BH, long Nq, long Nk, unsigned p8, uint32_t seed_lo, uint32_t seed_hi,
                        uint32_t offset, unsigned char *keep);
int oracle_bwd_heads(const double *q, const double *k, const double *v, const double *dout, long B,
                     long H, long N, long d, double scale, int causal, const long *heads, long nheads,
                     double *dq, double *dk, double *dv, int nthreads);
int oracle_bwd(const double *q, const double *k, const double *v, const double *dout, long B, long H,
               long N, long d, double scale, int causal, double *dq, double *dk, double *dv,
               int nthreads);
int oracle_fwd_padded(const double *q, const double *k, const double *v, long B, long H, long Nq,
                      long Nk, long d, const long *lq, const long *lk, double scale, int causal,
                      unsigned p8, uint32_t seed_lo, uint32_t seed_hi, uint32_t offset, double *o,
                      double *lse);
int oracle_bwd_padded(const double *q, const double *k, const double *v, const double *dout, long B,
                      long H, long Nq, long Nk, long d, const long *lq, const long *lk, double scale,
                      int causal, unsigned p8, uint32_t seed_lo, uint32_t seed_hi, uint32_t offset,
                      double *dq, double *dk, double *dv, int nthreads);

static int failures = 0;

#define CHECK(cond, ...)                     \
  do {                                       \
    if (!(cond)) {                           \
      fprintf(stderr, "FAIL %s:%d: ", __FILE__, __LINE__); \
      fprintf(stderr, __VA_ARGS__);          \
      fputc('\n', stderr);                   \
      ++failures;                            \
    }                                        \
  } while (0)

/* exact-size buffer of n doubles in [-2, 2) from a fixed linear congruence */
static double *filled(long n, uint64_t seed) {
  double *p = (double *)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  uint64_t x = seed * 6364136223846793005ULL + 1442695040888963407ULL;
  for (long i = 0; i < n; ++i) {
    x = x * 6364136223846793005ULL + 1442695040888963407ULL;
    p[i] = (double)(x >> 11) / 9007199254740992.0 * 4.0 - 2.0;
  }
  return p;
}

static int all_finite(const double *p, long n) {
  for (long i = 0; i < n; ++i)
    if (!isfinite(p[i])) return 0;
  return 1;
}

static void square_cases(void) {
  const long shapes[][4] = {{1, 1, 1, 1}, {1, 1, 1, 64}, {1, 2, 3, 2}, {2, 1, 17, 8}, {1, 1, 130, 128}};
  const double scales[] = {0.0, -0.7, 0.125, 3.0};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
    long B = shapes[s][0], H = shapes[s][1], N = shapes[s][2], d = shapes[s][3];
    long n = B * H * N * d, rows = B * H * N;
    double *q = filled(n, 1 + s), *k = filled(n, 11 + s), *v = filled(n, 21 + s), *dO = filled(n, 31 + s);
    for (int causal = 0; causal < 2; ++causal)
      for (size_t c = 0; c < sizeof scales / sizeof scales[0]; ++c)
        for (int threads = 0; threads <= 3; threads += 3) {
          double *o = filled(n, 0), *lse = filled(rows, 0);
          double *dq = filled(n, 0), *dk = filled(n, 0), *dv = filled(n, 0);
          int rc = oracle_fwd(q, k, v, B, H, N, d, scales[c], causal, o, lse, threads);
          CHECK(rc == 0 && all_finite(o, n) && all_finite(lse, rows), "fwd B%ld H%ld N%ld d%ld rc %d", B, H, N, d, rc);
          rc = oracle_bwd(q, k, v, dO, B, H, N, d, scales[c], causal, dq, dk, dv, threads);
          CHECK(rc == 0 && all_finite(dq, n) && all_finite(dk, n) && all_finite(dv, n), "bwd N%ld rc %d", N, rc);
          free(o); free(lse); free(dq); free(dk); free(dv);
        }
    /* a row subset, the empty subset, rows out of range, one head */
    long sel[3] = {rows - 1, 0, rows / 2};
    double *o3 = filled(3 * d, 0), *l3 = filled(3, 0);
    CHECK(oracle_fwd_rows(q, k, v, B, H, N, d, 0.5, 1, sel, 3, o3, l3, 2) == 0, "rows");
    CHECK(oracle_fwd_rows(q, k, v, B, H, N, d, 0.5, 1, sel, 0, o3, l3, 2) == 0, "no rows");
    long bad[1] = {rows};
    CHECK(oracle_fwd_rows(q, k, v, B, H, N, d, 0.5, 1, bad, 1, o3, l3, 2) == 3, "row out of range");
    bad[0] = -1;
    CHECK(oracle_fwd_rows(q, k, v, B, H, N, d, 0.5, 1, bad, 1, o3, l3, 2) == 3, "negative row");
    long head[1] = {B * H - 1};
    double *hq = filled(N * d, 0), *hk = filled(N * d, 0), *hv = filled(N * d, 0);
    CHECK(oracle_bwd_heads(q, k, v, dO, B, H, N, d, 0.5, 1, head, 1, hq, hk, hv, 64) == 0, "one head");
    head[0] = B * H;
    CHECK(oracle_bwd_heads(q, k, v, dO, B, H, N, d, 0.5, 1, head, 1, hq, hk, hv, 1) == 3, "head out of range");
    free(o3); free(l3); free(hq); free(hk); free(hv);
    free(q); free(k); free(v); free(dO);
  }
  /* argument errors */
  double x[4] = {0, 0, 0, 0};
  CHECK(oracle_fwd(NULL, x, x, 1, 1, 1, 1, 1.0, 0, x, x, 1) == 1, "null q");
  CHECK(oracle_fwd(x, x, x, 0, 1, 1, 1, 1.0, 0, x, x, 1) == 2, "B = 0");
  CHECK(oracle_bwd(x, x, x, x, 1, 1, 1, 0, 1.0, 0, x, x, x, 1) == 2, "d = 0");
}

static void padded_cases(void) {
  /* (Nq, Nk, lq[3], lk[3]) with empty, full and partial lengths */
  const long cases[][8] = {
      {5, 7, 5, 0, 3, 7, 4, 0}, {7, 5, 0, 7, 2, 5, 5, 1}, {1, 9, 1, 1, 0, 9, 1, 9}, {33, 33, 33, 17, 1, 33, 33, 2},
  };
  const unsigned p8s[] = {0, 26, 255};
  const long B = 3, H = 2, d = 4;
  for (size_t c = 0; c < sizeof cases / sizeof cases[0]; ++c) {
    long Nq = cases[c][0], Nk = cases[c][1];
    long lq[3] = {cases[c][2], cases[c][3], cases[c][4]}, lk[3] = {cases[c][5], cases[c][6], cases[c][7]};
    long nq = B * H * Nq * d, nk = B * H * Nk * d;
    double *q = filled(nq, 41 + c), *k = filled(nk, 51 + c), *v = filled(nk, 61 + c), *dO = filled(nq, 71 + c);
    for (int causal = 0; causal < 2; ++causal)
      for (size_t p = 0; p < sizeof p8s / sizeof p8s[0]; ++p) {
        double *o = filled(nq, 0), *lse = filled(B * H * Nq, 0);
        double *dq = filled(nq, 0), *dk = filled(nk, 0), *dv = filled(nk, 0);
        int rc = oracle_fwd_padded(q, k, v, B, H, Nq, Nk, d, lq, lk, 0.5, causal, p8s[p], 7, 9, 3, o, lse);
        CHECK(rc == 0, "padded fwd rc %d", rc);
        for (long b = 0; b < B; ++b)
          for (long h = 0; h < H; ++h)
            for (long i = 0; i < Nq; ++i) {
              const long r = (b * H + h) * Nq + i;
              /* a row sees a key iff it is valid, Lk > 0 and (causal) i + Lk - Lq >= 0 */
              const int sees = i < lq[b] && lk[b] > 0 && (!causal || i + lk[b] - lq[b] >= 0);
              CHECK(sees ? isfinite(lse[r]) : (isinf(lse[r]) && lse[r] < 0), "lse row %ld", r);
              if (!sees)
                for (long e = 0; e < d; ++e) CHECK(o[r * d + e] == 0.0, "dead row %ld", r);
            }
        rc = oracle_bwd_padded(q, k, v, dO, B, H, Nq, Nk, d, lq, lk, 0.5, causal, p8s[p], 7, 9, 3, dq, dk,
                               dv, 2);
        CHECK(rc == 0 && all_finite(dq, nq) && all_finite(dk, nk) && all_finite(dv, nk), "padded bwd rc %d", rc);
        free(o); free(lse); free(dq); free(dk); free(dv);
      }
    /* NULL lengths (all valid), lengths out of range, p8 out of range */
    double *o = filled(nq, 0), *lse = filled(B * H * Nq, 0);
    CHECK(oracle_fwd_padded(q, k, v, B, H, Nq, Nk, d, NULL, NULL, 0.5, 1, 0, 0, 0, 0, o, lse) == 0, "null lengths");
    long over[3] = {Nq + 1, 0, 0};
    CHECK(oracle_fwd_padded(q, k, v, B, H, Nq, Nk, d, over, NULL, 0.5, 1, 0, 0, 0, 0, o, lse) == 3, "lq > Nq");
    long neg[3] = {0, -1, 0};
    CHECK(oracle_fwd_padded(q, k, v, B, H, Nq, Nk, d, NULL, neg, 0.5, 1, 0, 0, 0, 0, o, lse) == 3, "lk < 0");
    CHECK(oracle_fwd_padded(q, k, v, B, H, Nq, Nk, d, NULL, NULL, 0.5, 1, 256, 0, 0, 0, o, lse) == 3, "p8 256");
    free(o); free(lse);
    free(q); free(k); free(v); free(dO);
  }
}

static void dropout_cases(void) {
  const long BH = 2, Nq = 5, Nk = 9;
  unsigned char *keep = (unsigned char *)malloc((size_t)(BH * Nq * Nk));
  CHECK(oracle_dropout_mask(BH, Nq, Nk, 0, 1, 2, 3, keep) == 0, "p8 0");
  for (long i = 0; i < BH * Nq * Nk; ++i) CHECK(keep[i] == 1, "p8 = 0 keeps every pair");
  CHECK(oracle_dropout_mask(BH, Nq, Nk, 255, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, keep) == 0, "p8 255");
  CHECK(oracle_dropout_mask(BH, Nq, Nk, 256, 1, 2, 3, keep) == 1, "p8 256 rejected");
  free(keep);
  uint32_t ctr[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu}, key[2] = {0xFFFFFFFFu, 0xFFFFFFFFu}, out[4];
  oracle_philox4x32_10(ctr, key, out);
}

int main(void) {
  square_cases();
  padded_cases();
  dropout_cases();
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle edge cases: all passed\n");
  return 0;
}
