/*
 * Exact softmax attention in fp64 on the CPU -- the correctness oracle.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path links, loads or calls
 * this file; only the test suite, the smoke check and the CPU-baseline leg of
 * the benchmark do.  It shares no code, header or constant with the HIP kernels.
 *
 * What it computes (the plain, materialised definition, no tiling, no online
 * rescaling):
 *   - "FlashAttention: lightning-fast Transformer" (llmtrend.com), section on the
 *     bottleneck of self-attention: Attention(Q,K,V) = softmax(Q K^T / sqrt(d_k)) V,
 *     evaluated in its four listed steps (similarities, scaling, softmax, weighted
 *     sum of V).  The scale is an argument; callers pass 1/sqrt(d) by default.
 *   - "MHA tuning, part 1" (handbook ch.3), section "where is the memory bottleneck
 *     of classic MHA": the eager form scores = Q K^T * scale, weights = softmax,
 *     output = weights V, with the score tensor shaped [batch, heads, seq, seq].
 *   - Same page, section "engineering implementation": the per-row log-sum-exp
 *     statistic kept beside the output (natural log of the sum of exp of the
 *     scaled, masked scores).
 *   - Same page, section "notes in practice" (causal mask: future positions are
 *     skipped).  Query i sees key j iff j <= i (square, top-left aligned).
 *   - llmtrend.com, "numerical stability": subtract the row max before exp.
 *   - "Flash Attention application" (jsqmd.com), section "Recomputation": the
 *     backward does not keep P from the forward; here P is recomputed from the
 *     inputs.  The gradient formulas are the calculus of the definition above
 *     (the pages print none):
 *       dV_j  = sum_i P_ij dO_i
 *       dP_ij = dO_i . V_j
 *       D_i   = sum_j P_ij dP_ij
 *       dS_ij = P_ij (dP_ij - D_i)
 *       dQ_i  = scale * sum_j dS_ij K_j
 *       dK_j  = scale * sum_i dS_ij Q_i
 *
 * Layout: Q,K,V,O,dO,dQ,dK,dV are contiguous [B][H][N][d] arrays of double;
 * LSE is [B][H][N].  Rows of one head are split across pthreads; each row's full
 * score vector is formed (a row of the N x N matrix), so the result does not
 * depend on the thread count.
 *
 * Padded batches and cross-attention (oracle_fwd_padded, oracle_bwd_padded):
 * Q, O, dO, dQ are [B][H][Nq][d], K, V, dK, dV are [B][H][Nk][d], and batch b
 * has Lq[b] <= Nq valid queries and Lk[b] <= Nk valid keys (the padding mask
 * that "Flash Attention application" (jsqmd.com), section "Notes", recommends
 * beside the causal one; cross-attention with its own key length is the case
 * llmtrend.com's "Limitations" section says needs a separate implementation).
 * Valid query i sees valid key j iff !causal or j <= i + Lk - Lq: the causal
 * diagonal is aligned to the last query and the last key, which for Lq = Lk is
 * the square rule above.  A row with no visible key and every padding row has
 * O = 0 and LSE = -inf and contributes nothing to the gradients.
 *
 * Dropout on the attention weights ("MHA tuning, part 1", section "notes in
 * practice": the dropout mask has to be generated block by block during the
 * fused computation, so the backward regenerates the same mask).  With drop
 * threshold p8 in [0, 255] (drop probability p8 / 256), pair (i, j) of head
 * bh = b*H + h is kept iff byte (j mod 4) of word (i mod 4) of
 *   Philox4x32-10(counter = (j / 4, i / 4, bh, offset), key = (seed_lo, seed_hi))
 * is >= p8, and kept weights are scaled by 256 / (256 - p8):
 *   O_i = sum_j P_ij Z_ij V_j,  Z_ij = keep_ij * 256 / (256 - p8).
 * P (and so LSE) is the softmax before dropout.  Gradients:
 *   dV_j = sum_i P_ij Z_ij dO_i, dP_ij = Z_ij (dO_i . V_j), D_i = sum_j P_ij dP_ij,
 *   dS_ij = P_ij (dP_ij - D_i), dQ, dK as above.
 * Philox4x32-10 is the counter-based generator of Salmon, Moraes, Dror and Shaw,
 * "Parallel random numbers: as easy as 1, 2, 3" (SC'11): ten rounds of two
 * 32x32->64-bit multiplications by 0xD2511F53 and 0xCD9E8D57 whose halves are
 * permuted and xored with the key, the key advanced by (0x9E3779B9, 0xBB67AE85)
 * between rounds.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_MAX_THREADS 256

/* ------------------------------------------------------------------------ */
/* forward                                                                    */
/* ------------------------------------------------------------------------ */

/* Number of keys visible to query i: keys 0 .. nvis-1 (see the header). */
static long visible_keys(long i, long Lq, long Lk, int causal) {
  if (i >= Lq) return 0; /* padding row */
  if (!causal) return Lk;
  long n = i + Lk - Lq + 1;
  return n < 0 ? 0 : (n > Lk ? Lk : n);
}

/* One query row over its visible keys 0..nvis-1: s_j = scale * q.k_j,
 * P = softmax(s), o = P V, lse = m + log(sum exp(s - m)); a row with no
 * visible key gets o = 0, lse = -inf.  `s` is scratch of length nvis. */
static void fwd_row(const double *q, const double *K, const double *V, long nvis,
                    long d, double scale, const double *z, double *o, double *lse,
                    double *s) {
  if (nvis == 0) {
    for (long c = 0; c < d; ++c) o[c] = 0.0;
    *lse = -INFINITY;
    return;
  }
  double m = -INFINITY;
  for (long j = 0; j < nvis; ++j) {
    double acc = 0.0;
    for (long c = 0; c < d; ++c) acc += q[c] * K[j * d + c];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (long j = 0; j < nvis; ++j) {
    s[j] = exp(s[j] - m); /* unnormalised weight */
    l += s[j];
  }
  for (long c = 0; c < d; ++c) o[c] = 0.0;
  for (long j = 0; j < nvis; ++j) {
    double p = s[j] / l;
    if (z) p *= z[j]; /* dropout multiplier (0 or 256 / (256 - p8)) */
    for (long c = 0; c < d; ++c) o[c] += p * V[j * d + c];
  }
  *lse = m + log(l);
}

typedef struct {
  const double *q, *k, *v;
  long H, N, d;
  double scale;
  int causal;
  const long *rows; /* flat row ids b*H*N + h*N + i */
  long nrows;
  double *o, *lse; /* per selected row: o[r*d..], lse[r] */
  long r0, r1;
} fwd_job;

static void *fwd_worker(void *arg) {
  fwd_job *J = (fwd_job *)arg;
  double *s = (double *)malloc(sizeof(double) * (size_t)J->N);
  if (!s) return (void *)1;
  for (long r = J->r0; r < J->r1; ++r) {
    long flat = J->rows[r];
    long bh = flat / J->N, i = flat % J->N;
    const double *Kh = J->k + bh * J->N * J->d;
    const double *Vh = J->v + bh * J->N * J->d;
    fwd_row(J->q + flat * J->d, Kh, Vh, visible_keys(i, J->N, J->N, J->causal), J->d,
            J->scale, NULL, J->o + r * J->d, J->lse + r, s);
  }
  free(s);
  return NULL;
}

static int clamp_threads(int t) {
  if (t < 1) return 1;
  if (t > ORACLE_MAX_THREADS) return ORACLE_MAX_THREADS;
  return t;
}

/* Forward on a chosen set of query rows.  rows[r] = b*H*N + h*N + i.
 * Returns 0 on success, nonzero on bad arguments or allocation failure. */
int oracle_fwd_rows(const double *q, const double *k, const double *v, long B,
                    long H, long N, long d, double scale, int causal,
                    const long *rows, long nrows, double *o_rows,
                    double *lse_rows, int nthreads) {
  if (!q || !k || !v || !rows || !o_rows || !lse_rows) return 1;
  if (B < 1 || H < 1 || N < 1 || d < 1 || nrows < 0) return 2;
  for (long r = 0; r < nrows; ++r)
    if (rows[r] < 0 || rows[r] >= B * H * N) return 3;
  int T = clamp_threads(nthreads);
  if (T > nrows) T = nrows > 0 ? (int)nrows : 1;
  pthread_t th[ORACLE_MAX_THREADS];
  fwd_job jobs[ORACLE_MAX_THREADS];
  int err = 0;
  for (int t = 0; t < T; ++t) {
    fwd_job *J = &jobs[t];
    J->q = q; J->k = k; J->v = v; J->H = H; J->N = N; J->d = d;
    J->scale = scale; J->causal = causal; J->rows = rows; J->nrows = nrows;
    J->o = o_rows; J->lse = lse_rows;
    J->r0 = nrows * t / T; J->r1 = nrows * (t + 1) / T;
  }
  for (int t = 1; t < T; ++t)
    if (pthread_create(&th[t], NULL, fwd_worker, &jobs[t])) err = 4;
  if (fwd_worker(&jobs[0])) err = 5;
  for (int t = 1; t < T; ++t) {
    void *ret = NULL;
    pthread_join(th[t], &ret);
    if (ret) err = 5;
  }
  return err;
}

/* Forward over every row of every head. */
int oracle_fwd(const double *q, const double *k, const double *v, long B,
               long H, long N, long d, double scale, int causal, double *o,
               double *lse, int nthreads) {
  long total = B * H * N;
  if (total < 1) return 2;
  long *rows = (long *)malloc(sizeof(long) * (size_t)total);
  if (!rows) return 5;
  for (long r = 0; r < total; ++r) rows[r] = r;
  int rc = oracle_fwd_rows(q, k, v, B, H, N, d, scale, causal, rows, total, o,
                           lse, nthreads);
  free(rows);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* dropout mask: Philox4x32-10 (see the header)                               */
/* ------------------------------------------------------------------------ */

void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  uint32_t x[4] = {ctr[0], ctr[1], ctr[2], ctr[3]};
  uint32_t k[2] = {key[0], key[1]};
  for (int round = 0; round < 10; ++round) {
    if (round > 0) { /* key schedule: a Weyl sequence */
      k[0] += 0x9E3779B9u;
      k[1] += 0xBB67AE85u;
    }
    uint64_t a = (uint64_t)0xD2511F53u * x[0];
    uint64_t b = (uint64_t)0xCD9E8D57u * x[2];
    uint32_t y0 = (uint32_t)(b >> 32) ^ x[1] ^ k[0];
    uint32_t y1 = (uint32_t)b;
    uint32_t y2 = (uint32_t)(a >> 32) ^ x[3] ^ k[1];
    uint32_t y3 = (uint32_t)a;
    x[0] = y0; x[1] = y1; x[2] = y2; x[3] = y3;
  }
  memcpy(out, x, sizeof x);
}

typedef struct {
  unsigned p8;       /* drop threshold 0..255; 0 = no dropout */
  uint32_t seed_lo, seed_hi, offset;
} dropout_spec;

/* Z_ij of pair (i, j) of head bh: 0 (dropped) or 256 / (256 - p8). */
static double dropout_mult(const dropout_spec *dr, long bh, long i, long j) {
  uint32_t ctr[4] = {(uint32_t)(j >> 2), (uint32_t)(i >> 2), (uint32_t)bh, dr->offset};
  uint32_t key[2] = {dr->seed_lo, dr->seed_hi};
  uint32_t r[4];
  oracle_philox4x32_10(ctr, key, r);
  unsigned byte = (r[i & 3] >> (8 * (j & 3))) & 0xFFu;
  return byte >= dr->p8 ? 256.0 / (256.0 - (double)dr->p8) : 0.0;
}

/* keep[bh][i][j] (0/1 bytes) for every pair of B*H heads of Nq x Nk. */
int oracle_dropout_mask(long BH, long Nq, long Nk, unsigned p8, uint32_t seed_lo,
                        uint32_t seed_hi, uint32_t offset, unsigned char *keep) {
  if (!keep || BH < 1 || Nq < 1 || Nk < 1 || p8 > 255) return 1;
  dropout_spec dr = {p8, seed_lo, seed_hi, offset};
  for (long bh = 0; bh < BH; ++bh)
    for (long i = 0; i < Nq; ++i)
      for (long j = 0; j < Nk; ++j)
        keep[(bh * Nq + i) * Nk + j] = dropout_mult(&dr, bh, i, j) != 0.0;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* backward, one head at a time, with the N x N matrices P and dS formed      */
/* ------------------------------------------------------------------------ */

typedef struct {
  const double *q, *dout;         /* this head, [Nq][d] */
  const double *k, *v;            /* this head, [Nk][d] */
  double *P, *dS;                 /* [Nq][Nk] */
  double *Z;                      /* [Nq][Nk] dropout multipliers, or NULL */
  const dropout_spec *drop;       /* used when Z != NULL */
  long bh;                        /* head index b*H + h (dropout counter) */
  double *dq;                     /* this head, [Nq][d] */
  double *dk, *dv;                /* this head, [Nk][d] */
  long Nq, Nk, Lq, Lk, d;         /* Lq, Lk: valid queries / keys of this batch entry */
  double scale;
  int causal;
  int phase;
  long a0, a1; /* row (phase 0, 2) or column (phase 1, 3) range */
} bwd_job;

static void *bwd_worker(void *arg) {
  bwd_job *J = (bwd_job *)arg;
  long Nq = J->Nq, Nk = J->Nk, d = J->d;
  if (J->phase == 0) {
    /* rows of P: recomputed from Q, K as in the forward */
    for (long i = J->a0; i < J->a1; ++i) {
      double *Pi = J->P + i * Nk;
      long nvis = visible_keys(i, J->Lq, J->Lk, J->causal);
      double m = -INFINITY;
      for (long j = 0; j < nvis; ++j) {
        double acc = 0.0;
        for (long c = 0; c < d; ++c) acc += J->q[i * d + c] * J->k[j * d + c];
        Pi[j] = J->scale * acc;
        if (Pi[j] > m) m = Pi[j];
      }
      double l = 0.0;
      for (long j = 0; j < nvis; ++j) {
        Pi[j] = exp(Pi[j] - m);
        l += Pi[j];
      }
      for (long j = 0; j < nvis; ++j) Pi[j] /= l;
      for (long j = nvis; j < Nk; ++j) Pi[j] = 0.0; /* masked: weight 0 */
      if (J->Z)
        for (long j = 0; j < Nk; ++j) J->Z[i * Nk + j] = dropout_mult(J->drop, J->bh, i, j);
    }
  } else if (J->phase == 1) {
    /* dV_j = sum_i P_ij Z_ij dO_i */
    for (long j = J->a0; j < J->a1; ++j)
      for (long c = 0; c < d; ++c) {
        double acc = 0.0;
        for (long i = 0; i < Nq; ++i) {
          double w = J->P[i * Nk + j];
          if (J->Z) w *= J->Z[i * Nk + j];
          acc += w * J->dout[i * d + c];
        }
        J->dv[j * d + c] = acc;
      }
  } else if (J->phase == 2) {
    /* dP_ij = dO_i . V_j ; D_i = sum_j P_ij dP_ij ; dS = P (dP - D) ;
     * dQ_i = scale * sum_j dS_ij K_j */
    for (long i = J->a0; i < J->a1; ++i) {
      double *dSi = J->dS + i * Nk;
      const double *Pi = J->P + i * Nk;
      for (long j = 0; j < Nk; ++j) {
        double acc = 0.0;
        for (long c = 0; c < d; ++c) acc += J->dout[i * d + c] * J->v[j * d + c];
        if (J->Z) acc *= J->Z[i * Nk + j];
        dSi[j] = acc; /* dP for now */
      }
      double D = 0.0;
      for (long j = 0; j < Nk; ++j) D += Pi[j] * dSi[j];
      for (long j = 0; j < Nk; ++j) dSi[j] = Pi[j] * (dSi[j] - D);
      for (long c = 0; c < d; ++c) {
        double acc = 0.0;
        for (long j = 0; j < Nk; ++j) acc += dSi[j] * J->k[j * d + c];
        J->dq[i * d + c] = J->scale * acc;
      }
    }
  } else {
    /* dK_j = scale * sum_i dS_ij Q_i */
    for (long j = J->a0; j < J->a1; ++j)
      for (long c = 0; c < d; ++c) {
        double acc = 0.0;
        for (long i = 0; i < Nq; ++i) acc += J->dS[i * Nk + j] * J->q[i * d + c];
        J->dk[j * d + c] = J->scale * acc;
      }
  }
  return NULL;
}

static int run_phase(bwd_job *base, int phase, int T) {
  pthread_t th[ORACLE_MAX_THREADS];
  bwd_job jobs[ORACLE_MAX_THREADS];
  int err = 0;
  long n = (phase == 0 || phase == 2) ? base->Nq : base->Nk; /* rows or columns */
  for (int t = 0; t < T; ++t) {
    jobs[t] = *base;
    jobs[t].phase = phase;
    jobs[t].a0 = n * t / T;
    jobs[t].a1 = n * (t + 1) / T;
  }
  for (int t = 1; t < T; ++t)
    if (pthread_create(&th[t], NULL, bwd_worker, &jobs[t])) err = 4;
  bwd_worker(&jobs[0]);
  for (int t = 1; t < T; ++t) pthread_join(th[t], NULL);
  return err;
}

/* Backward for a chosen set of heads.  heads[h] = b*H + h.  Outputs dq, dk, dv
 * are [nheads][N][d] (one block per selected head, in the order given).
 * The four phases run one after another; each needs the previous phase's
 * matrices complete.  Returns 0 on success. */
int oracle_bwd_heads(const double *q, const double *k, const double *v,
                     const double *dout, long B, long H, long N, long d,
                     double scale, int causal, const long *heads, long nheads,
                     double *dq, double *dk, double *dv, int nthreads) {
  if (!q || !k || !v || !dout || !heads || !dq || !dk || !dv) return 1;
  if (B < 1 || H < 1 || N < 1 || d < 1 || nheads < 0) return 2;
  for (long x = 0; x < nheads; ++x)
    if (heads[x] < 0 || heads[x] >= B * H) return 3;
  int T = clamp_threads(nthreads);
  if (T > N) T = (int)N;
  double *P = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
  double *dS = (double *)malloc(sizeof(double) * (size_t)N * (size_t)N);
  if (!P || !dS) {
    free(P);
    free(dS);
    return 5;
  }
  int err = 0;
  for (long x = 0; x < nheads && !err; ++x) {
    long off = heads[x] * N * d;
    bwd_job base;
    memset(&base, 0, sizeof base);
    base.q = q + off; base.k = k + off; base.v = v + off; base.dout = dout + off;
    base.P = P; base.dS = dS;
    base.dq = dq + x * N * d; base.dk = dk + x * N * d; base.dv = dv + x * N * d;
    base.Nq = N; base.Nk = N; base.Lq = N; base.Lk = N;
    base.d = d; base.scale = scale; base.causal = causal;
    for (int phase = 0; phase < 4 && !err; ++phase) err = run_phase(&base, phase, T);
  }
  free(P);
  free(dS);
  return err;
}

/* Backward over every head. */
int oracle_bwd(const double *q, const double *k, const double *v,
               const double *dout, long B, long H, long N, long d, double scale,
               int causal, double *dq, double *dk, double *dv, int nthreads) {
  long nh = B * H;
  if (nh < 1) return 2;
  long *heads = (long *)malloc(sizeof(long) * (size_t)nh);
  if (!heads) return 5;
  for (long x = 0; x < nh; ++x) heads[x] = x;
  int rc = oracle_bwd_heads(q, k, v, dout, B, H, N, d, scale, causal, heads, nh,
                            dq, dk, dv, nthreads);
  free(heads);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* padded batches and cross-attention (see the header)                        */
/* ------------------------------------------------------------------------ */

/* Lengths: lq[b] in [0, Nq], lk[b] in [0, Nk]; NULL means all valid. */
static int lengths_ok(const long *lq, const long *lk, long B, long Nq, long Nk) {
  for (long b = 0; b < B; ++b) {
    if (lq && (lq[b] < 0 || lq[b] > Nq)) return 0;
    if (lk && (lk[b] < 0 || lk[b] > Nk)) return 0;
  }
  return 1;
}

/* Forward over every row: o [B][H][Nq][d], lse [B][H][Nq]. */
int oracle_fwd_padded(const double *q, const double *k, const double *v, long B,
                      long H, long Nq, long Nk, long d, const long *lq,
                      const long *lk, double scale, int causal, unsigned p8,
                      uint32_t seed_lo, uint32_t seed_hi, uint32_t offset, double *o,
                      double *lse) {
  if (!q || !k || !v || !o || !lse) return 1;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return 2;
  if (!lengths_ok(lq, lk, B, Nq, Nk) || p8 > 255) return 3;
  dropout_spec dr = {p8, seed_lo, seed_hi, offset};
  double *s = (double *)malloc(sizeof(double) * (size_t)Nk);
  double *z = p8 ? (double *)malloc(sizeof(double) * (size_t)Nk) : NULL;
  if (!s || (p8 && !z)) {
    free(s);
    free(z);
    return 5;
  }
  for (long b = 0; b < B; ++b) {
    long Lq = lq ? lq[b] : Nq, Lk = lk ? lk[b] : Nk;
    for (long h = 0; h < H; ++h) {
      long bh = b * H + h;
      for (long i = 0; i < Nq; ++i) {
        if (z)
          for (long j = 0; j < Nk; ++j) z[j] = dropout_mult(&dr, bh, i, j);
        fwd_row(q + (bh * Nq + i) * d, k + bh * Nk * d, v + bh * Nk * d,
                visible_keys(i, Lq, Lk, causal), d, scale, z, o + (bh * Nq + i) * d,
                lse + bh * Nq + i, s);
      }
    }
  }
  free(s);
  free(z);
  return 0;
}

/* Backward over every head: dq [B][H][Nq][d], dk and dv [B][H][Nk][d]. */
int oracle_bwd_padded(const double *q, const double *k, const double *v,
                      const double *dout, long B, long H, long Nq, long Nk, long d,
                      const long *lq, const long *lk, double scale, int causal,
                      unsigned p8, uint32_t seed_lo, uint32_t seed_hi, uint32_t offset,
                      double *dq, double *dk, double *dv, int nthreads) {
  if (!q || !k || !v || !dout || !dq || !dk || !dv) return 1;
  if (B < 1 || H < 1 || Nq < 1 || Nk < 1 || d < 1) return 2;
  if (!lengths_ok(lq, lk, B, Nq, Nk) || p8 > 255) return 3;
  dropout_spec dr = {p8, seed_lo, seed_hi, offset};
  int T = clamp_threads(nthreads);
  if (T > Nq) T = (int)Nq;
  if (T > Nk) T = (int)Nk;
  double *P = (double *)malloc(sizeof(double) * (size_t)Nq * (size_t)Nk);
  double *dS = (double *)malloc(sizeof(double) * (size_t)Nq * (size_t)Nk);
  double *Z = p8 ? (double *)malloc(sizeof(double) * (size_t)Nq * (size_t)Nk) : NULL;
  if (!P || !dS || (p8 && !Z)) {
    free(P);
    free(dS);
    free(Z);
    return 5;
  }
  int err = 0;
  for (long bh = 0; bh < B * H && !err; ++bh) {
    long b = bh / H;
    bwd_job base;
    memset(&base, 0, sizeof base);
    base.q = q + bh * Nq * d; base.dout = dout + bh * Nq * d;
    base.k = k + bh * Nk * d; base.v = v + bh * Nk * d;
    base.P = P; base.dS = dS;
    base.dq = dq + bh * Nq * d; base.dk = dk + bh * Nk * d; base.dv = dv + bh * Nk * d;
    base.Nq = Nq; base.Nk = Nk; base.Lq = lq ? lq[b] : Nq; base.Lk = lk ? lk[b] : Nk;
    base.d = d; base.scale = scale; base.causal = causal;
    base.Z = Z; base.drop = &dr; base.bh = bh;
    for (int phase = 0; phase < 4 && !err; ++phase) err = run_phase(&base, phase, T);
  }
  free(P);
  free(dS);
  free(Z);
  return err;
}
