/*
 * oracle.c -- plain, slow, fp64 CPU reference for exact attention.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * bench's CPU-baseline leg may load this library.  It shares no code with the
 * GPU library and must never be used as a fallback for it.
 *
 * What it computes is the textbook definition that the tiled method reaches
 * exactly, up to the order of floating-point additions ("S12 FlashAttention",
 * llminference.xinbetween.com, sections "Motivation / The problem" and "What
 * this unlocks beyond speed"): for one query row i of one head,
 *
 *     s_j   = scale * sum_c q[i][c] * k[j][c]        for every visible key j
 *     M     = max_j s_j
 *     Z     = sum_j exp(s_j - M)
 *     O[i]  = (sum_j exp(s_j - M) * v[j]) / Z
 *     LSE_i = M + ln Z                                 (natural log)
 *
 * The whole score row s is materialised in a scratch array before the softmax
 * (S is never tiled here).  Everything is double precision; inputs may be
 * double, float or bf16 bit patterns and are widened exactly, element by
 * element.  A row with no visible key gets O = 0 and LSE = -inf.
 *
 * Visible keys:
 *   - non-causal: every key;
 *   - causal: key j is visible from query i iff j <= i + (Nk - Nq)  (queries
 *     aligned to the end of the keys; identical to j <= i when Nq == Nk);
 *   - packed variable length ("FlashAttention: The Algorithm That Beat the
 *     Memory Wall", repo-explainer.com, section "Varlen Is the Quiet
 *     Superpower"): only keys of the query's own sequence, causal in local
 *     positions;
 *   - paged decode ("S12 FlashAttention", section "Build it / Implementation",
 *     the paged excerpt, and "How this composes with what you already built"):
 *     logical key t of sequence b is pool[block_table[b][t / block]][g][t % block]
 *     with g = h / (Hq / Hkv), for t < seq_len[b].
 *
 * Dropout of the normalised weights (the *_dropout entry points) is described
 * at dropout_t below; the generator it draws from is Philox-4x32-10, written
 * from its published definition and pinned to the published known answers.
 *
 * Status codes: 0 ok, 1 bad argument, 2 out of memory.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F64 = 0, ORC_F32 = 1, ORC_BF16 = 2 };

/* Widen element i of a typed buffer to double, exactly. */
static double load(const void *p, int dtype, int64_t i) {
  if (dtype == ORC_F64) return ((const double *)p)[i];
  if (dtype == ORC_F32) return (double)((const float *)p)[i];
  uint32_t bits = (uint32_t)((const uint16_t *)p)[i] << 16;
  float f;
  memcpy(&f, &bits, sizeof f);
  return (double)f;
}

/*
 * Philox-4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC 2011): ten rounds on a 4-word counter under a 2-word
 * key.  A round multiplies counter words 0 and 2 by M0 and M1 into 64-bit
 * products and forms {hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0}; between rounds
 * the key words advance by W0 and W1.
 */
void oracle_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]) {
  const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u, W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3], k0 = key[0], k1 = key[1];
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += W0;
      k1 += W1;
    }
    const uint64_t p0 = (uint64_t)M0 * c0, p1 = (uint64_t)M1 * c2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    c0 = hi1 ^ c1 ^ k0;
    c1 = lo1;
    c2 = hi0 ^ c3 ^ k1;
    c3 = lo0;
  }
  out[0] = c0, out[1] = c1, out[2] = c2, out[3] = c3;
}

/*
 * Attention dropout ("FlashAttention: The Algorithm That Beat the Memory
 * Wall", repo-explainer.com, "How the Repo Connects Python to Bare-Metal
 * CUDA" and "Why Templates Matter Here" name dropout among the kernel's
 * parameters and specialisations; what it computes is the usual reading):
 * each normalised weight of row `row` and key j is kept with probability
 * (256 - t) / 256 and scaled by 256 / (256 - t), else zeroed; the LSE is
 * that of the weights before dropout.  The keep decision for (row, j) is
 * byte j % 16 (little-endian) of the Philox-4x32-10 output for counter
 * {j / 16, row low word, row high word, offset} and key {seed low, seed
 * high}: keep iff that byte >= t.
 */
typedef struct {
  int threshold; /* t in [0, 255]; 0 keeps everything */
  uint64_t seed;
  uint32_t offset;
  int64_t row; /* the row's id (its index in the LSE layout) */
} dropout_t;

static int dropout_keep(const dropout_t *dp, int64_t j) {
  const uint32_t ctr[4] = {(uint32_t)(j / 16), (uint32_t)dp->row, (uint32_t)((uint64_t)dp->row >> 32),
                           dp->offset};
  const uint32_t key[2] = {(uint32_t)dp->seed, (uint32_t)(dp->seed >> 32)};
  uint32_t out[4];
  oracle_philox4x32_10(ctr, key, out);
  const uint32_t byte = (out[(j % 16) / 4] >> (8 * (j % 4))) & 0xFFu;
  return (int)byte >= dp->threshold;
}

static void attend_row_dropout(const void *q, const void *k, const void *v, int dtype, int d,
                               double scale, int64_t qoff, const int64_t *koff,
                               const int64_t *voff, int64_t n, double *s, double *o,
                               double *lse, const dropout_t *dp);

/*
 * One query row against an explicit list of key/value row offsets.
 *   qoff        : element offset of the query row in q
 *   koff[j]     : element offset of key row j in k, voff[j] likewise in v
 *   n           : number of visible keys
 *   s           : scratch of n doubles (the materialised score row)
 *   o (d), lse  : outputs
 */
static void attend_row(const void *q, const void *k, const void *v, int dtype, int d,
                       double scale, int64_t qoff, const int64_t *koff,
                       const int64_t *voff, int64_t n, double *s, double *o,
                       double *lse) {
  attend_row_dropout(q, k, v, dtype, d, scale, qoff, koff, voff, n, s, o, lse, NULL);
}

/* attend_row with optional dropout of the normalised weights (dp may be NULL). */
static void attend_row_dropout(const void *q, const void *k, const void *v, int dtype, int d,
                               double scale, int64_t qoff, const int64_t *koff,
                               const int64_t *voff, int64_t n, double *s, double *o,
                               double *lse, const dropout_t *dp) {
  for (int c = 0; c < d; ++c) o[c] = 0.0;
  if (n <= 0) {
    *lse = -INFINITY;
    return;
  }
  /* S row: scaled dot products. */
  for (int64_t j = 0; j < n; ++j) {
    double acc = 0.0;
    for (int c = 0; c < d; ++c) acc += load(q, dtype, qoff + c) * load(k, dtype, koff[j] + c);
    s[j] = scale * acc;
  }
  /* Row maximum. */
  double m = s[0];
  for (int64_t j = 1; j < n; ++j)
    if (s[j] > m) m = s[j];
  /* Unnormalised weights and their sum. */
  double z = 0.0;
  for (int64_t j = 0; j < n; ++j) {
    s[j] = exp(s[j] - m);
    z += s[j];
  }
  /* Weighted sum of values (dropout: kept weights rescaled, dropped ones
   * zero), then normalise by the full sum. */
  const double keep_scale = dp ? 256.0 / (256 - dp->threshold) : 1.0;
  for (int64_t j = 0; j < n; ++j) {
    const double w = dp ? (dropout_keep(dp, j) ? s[j] * keep_scale : 0.0) : s[j];
    for (int c = 0; c < d; ++c) o[c] += w * load(v, dtype, voff[j] + c);
  }
  for (int c = 0; c < d; ++c) o[c] /= z;
  *lse = m + log(z);
}

static int set_threads(int nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
  return omp_get_max_threads();
#else
  (void)nthreads;
  return 1;
#endif
}

int oracle_max_threads(int nthreads) { return set_threads(nthreads); }

/*
 * FP8 E4M3 codes to their values ("S12 FlashAttention", "Production notes /
 * In production": FlashAttention-3 adds FP8 inputs; the format itself is the
 * OCP 8-bit floating point E4M3 format, which the pages do not restate):
 * bit 7 is the sign, bits 6..3 the exponent with bias 7, bits 2..0 the
 * mantissa.  Exponent 0 holds the subnormals m * 2^-9; exponent 15 with
 * mantissa 7 is NaN (there are no infinities), so the largest finite value
 * is 1.75 * 2^8 = 448.  Every value is exact in double.
 */
void oracle_decode_e4m3(const uint8_t *src, double *dst, int64_t n) {
  for (int64_t i = 0; i < n; ++i) {
    const int c = src[i];
    const int sign = c >> 7, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7)
      v = NAN;
    else if (e == 0)
      v = ldexp((double)m, -9);
    else
      v = ldexp(8.0 + m, e - 10); /* (1 + m/8) * 2^(e-7) */
    dst[i] = sign ? -v : v;
  }
}

/*
 * Dense batched attention.  q is [B, Nq, Hq, d], k and v are [B, Nk, Hkv, d],
 * addressed with element strides {batch, seq, head} (d is contiguous).
 * Rows are flattened ids r = (b * Hq + h) * Nq + i; rows == NULL means all
 * B*Hq*Nq rows in that order.  o is [nrows, d], lse is [nrows].
 */
static int dense_impl(const void *q, const void *k, const void *v, int dtype, int B, int Nq, int Nk,
                      int Hq, int Hkv, int d, const int64_t *qs, const int64_t *ks, const int64_t *vs,
                      int causal, double scale, const int64_t *rows, int64_t nrows, double *o,
                      double *lse, int nthreads, const dropout_t *drop);

int oracle_attn_dense(const void *q, const void *k, const void *v, int dtype, int B,
                      int Nq, int Nk, int Hq, int Hkv, int d, const int64_t *qs,
                      const int64_t *ks, const int64_t *vs, int causal, double scale,
                      const int64_t *rows, int64_t nrows, double *o, double *lse,
                      int nthreads) {
  return dense_impl(q, k, v, dtype, B, Nq, Nk, Hq, Hkv, d, qs, ks, vs, causal, scale, rows, nrows, o,
                    lse, nthreads, NULL);
}

/* Dense attention with dropout of the normalised weights (see dropout_t);
 * the row id of (b, h, i) is (b * Hq + h) * Nq + i. */
int oracle_attn_dense_dropout(const void *q, const void *k, const void *v, int dtype, int B,
                              int Nq, int Nk, int Hq, int Hkv, int d, const int64_t *qs,
                              const int64_t *ks, const int64_t *vs, int causal, double scale,
                              int threshold, uint64_t seed, uint32_t offset, const int64_t *rows,
                              int64_t nrows, double *o, double *lse, int nthreads) {
  if (threshold < 0 || threshold > 255) return 1;
  dropout_t drop = {threshold, seed, offset, 0};
  return dense_impl(q, k, v, dtype, B, Nq, Nk, Hq, Hkv, d, qs, ks, vs, causal, scale, rows, nrows, o,
                    lse, nthreads, &drop);
}

static int dense_impl(const void *q, const void *k, const void *v, int dtype, int B, int Nq, int Nk,
                      int Hq, int Hkv, int d, const int64_t *qs, const int64_t *ks, const int64_t *vs,
                      int causal, double scale, const int64_t *rows, int64_t nrows, double *o,
                      double *lse, int nthreads, const dropout_t *drop) {
  if (!q || !k || !v || !o || !lse || !qs || !ks || !vs) return 1;
  if (B < 0 || Nq < 0 || Nk < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv) return 1;
  if (!rows) nrows = (int64_t)B * Hq * Nq;
  if (Nq == 0 && nrows > 0) return 1;
  const int group = Hq / Hkv;
  int bad = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)(Nk > 0 ? Nk : 1));
    int64_t *koff = (int64_t *)malloc(sizeof(int64_t) * (size_t)(Nk > 0 ? Nk : 1));
    int64_t *voff = (int64_t *)malloc(sizeof(int64_t) * (size_t)(Nk > 0 ? Nk : 1));
    if (!s || !koff || !voff) {
#pragma omp atomic write
      bad = 2;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < nrows; ++r) {
        int64_t id = rows ? rows[r] : r;
        int64_t i = id % Nq, bh = id / Nq;
        int64_t h = bh % Hq, b = bh / Hq;
        if (id < 0 || b >= B) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        int64_t g = h / group;
        int64_t last = causal ? i + (Nk - Nq) : (int64_t)Nk - 1; /* last visible key */
        if (last > Nk - 1) last = Nk - 1;
        int64_t n = last + 1 > 0 ? last + 1 : 0;
        for (int64_t j = 0; j < n; ++j) {
          koff[j] = b * ks[0] + j * ks[1] + g * ks[2];
          voff[j] = b * vs[0] + j * vs[1] + g * vs[2];
        }
        dropout_t dp;
        if (drop) {
          dp = *drop;
          dp.row = id; /* (b * Hq + h) * Nq + i */
        }
        attend_row_dropout(q, k, v, dtype, d, scale, b * qs[0] + i * qs[1] + h * qs[2], koff, voff,
                           n, s, o + r * d, lse + r, drop ? &dp : NULL);
      }
    }
    free(s);
    free(koff);
    free(voff);
  }
  return bad;
}

/*
 * Packed variable-length attention.  q is [T, Hq, d], k and v [T, Hkv, d]
 * with element strides {token, head}; sequence s owns tokens
 * [cu[s], cu[s+1]).  Rows are flattened ids r = h * T + t (rows == NULL:
 * all Hq*T).  Keys are the query's own sequence, causal in local positions.
 */
static int varlen_impl(const void *q, const void *k, const void *v, int dtype, const int32_t *cu,
                       int nseq, int Hq, int Hkv, int d, const int64_t *qs, const int64_t *ks,
                       const int64_t *vs, int causal, double scale, const int64_t *rows,
                       int64_t nrows, double *o, double *lse, int nthreads, const dropout_t *drop);

int oracle_attn_varlen(const void *q, const void *k, const void *v, int dtype,
                       const int32_t *cu, int nseq, int Hq, int Hkv, int d,
                       const int64_t *qs, const int64_t *ks, const int64_t *vs, int causal,
                       double scale, const int64_t *rows, int64_t nrows, double *o,
                       double *lse, int nthreads) {
  return varlen_impl(q, k, v, dtype, cu, nseq, Hq, Hkv, d, qs, ks, vs, causal, scale, rows, nrows, o,
                     lse, nthreads, NULL);
}

/* Packed attention with dropout (see dropout_t); the row id of (h, token t)
 * is h * T + t, keys are numbered within their sequence. */
int oracle_attn_varlen_dropout(const void *q, const void *k, const void *v, int dtype,
                               const int32_t *cu, int nseq, int Hq, int Hkv, int d,
                               const int64_t *qs, const int64_t *ks, const int64_t *vs, int causal,
                               double scale, int threshold, uint64_t seed, uint32_t offset,
                               const int64_t *rows, int64_t nrows, double *o, double *lse,
                               int nthreads) {
  if (threshold < 0 || threshold > 255) return 1;
  dropout_t drop = {threshold, seed, offset, 0};
  return varlen_impl(q, k, v, dtype, cu, nseq, Hq, Hkv, d, qs, ks, vs, causal, scale, rows, nrows, o,
                     lse, nthreads, &drop);
}

static int varlen_impl(const void *q, const void *k, const void *v, int dtype, const int32_t *cu,
                       int nseq, int Hq, int Hkv, int d, const int64_t *qs, const int64_t *ks,
                       const int64_t *vs, int causal, double scale, const int64_t *rows,
                       int64_t nrows, double *o, double *lse, int nthreads, const dropout_t *drop) {
  if (!q || !k || !v || !cu || !o || !lse || !qs || !ks || !vs) return 1;
  if (nseq < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv) return 1;
  if (cu[0] != 0) return 1;
  for (int s = 0; s < nseq; ++s)
    if (cu[s + 1] < cu[s]) return 1;
  const int64_t T = cu[nseq];
  int64_t maxlen = 1;
  for (int s = 0; s < nseq; ++s)
    if (cu[s + 1] - cu[s] > maxlen) maxlen = cu[s + 1] - cu[s];
  if (!rows) nrows = (int64_t)Hq * T;
  const int group = Hq / Hkv;
  int bad = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)maxlen);
    int64_t *koff = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxlen);
    int64_t *voff = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxlen);
    if (!s || !koff || !voff) {
#pragma omp atomic write
      bad = 2;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < nrows; ++r) {
        int64_t id = rows ? rows[r] : r;
        int64_t t = id % (T > 0 ? T : 1), h = id / (T > 0 ? T : 1);
        if (id < 0 || h >= Hq || T == 0) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        int seq = 0;
        while (cu[seq + 1] <= t) ++seq; /* the sequence holding token t */
        int64_t start = cu[seq], len = cu[seq + 1] - cu[seq];
        int64_t i = t - start;
        int64_t n = causal ? i + 1 : len;
        int64_t g = h / group;
        for (int64_t j = 0; j < n; ++j) {
          koff[j] = (start + j) * ks[0] + g * ks[1];
          voff[j] = (start + j) * vs[0] + g * vs[1];
        }
        dropout_t dp;
        if (drop) {
          dp = *drop;
          dp.row = id; /* h * T + t */
        }
        attend_row_dropout(q, k, v, dtype, d, scale, t * qs[0] + h * qs[1], koff, voff, n, s,
                           o + r * d, lse + r, drop ? &dp : NULL);
      }
    }
    free(s);
    free(koff);
    free(voff);
  }
  return bad;
}

/*
 * Paged decode: one query token per sequence.  q is [B, Hq, d] (element
 * strides {batch, head}); the pools are addressed with element strides
 * {block, head, token}; block_table is [B, max_blocks] (row stride
 * max_blocks).  Rows are flattened ids r = b * Hq + h (rows == NULL: all).
 * The query of sequence b sees its seq_lens[b] logical keys.
 */
int oracle_attn_decode_paged(const void *q, const void *kpool, const void *vpool, int dtype,
                             const int64_t *qs, const int64_t *ps, const int32_t *block_table,
                             int max_blocks, const int32_t *seq_lens, int B, int Hq, int Hkv,
                             int d, int block_size, int num_blocks, double scale,
                             const int64_t *rows, int64_t nrows, double *o, double *lse,
                             int nthreads) {
  if (!q || !kpool || !vpool || !qs || !ps || !block_table || !seq_lens || !o || !lse) return 1;
  if (B < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv || block_size <= 0) return 1;
  int64_t maxlen = 1;
  for (int b = 0; b < B; ++b) {
    if (seq_lens[b] < 0 || (int64_t)seq_lens[b] > (int64_t)max_blocks * block_size) return 1;
    if (seq_lens[b] > maxlen) maxlen = seq_lens[b];
  }
  if (!rows) nrows = (int64_t)B * Hq;
  const int group = Hq / Hkv;
  int bad = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)maxlen);
    int64_t *koff = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxlen);
    if (!s || !koff) {
#pragma omp atomic write
      bad = 2;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t r = 0; r < nrows; ++r) {
        int64_t id = rows ? rows[r] : r;
        int64_t h = id % Hq, b = id / Hq;
        if (id < 0 || b >= B) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        int64_t g = h / group, n = seq_lens[b];
        int oob = 0;
        for (int64_t t = 0; t < n; ++t) {
          int64_t phys = block_table[b * (int64_t)max_blocks + t / block_size];
          if (phys < 0 || phys >= num_blocks) oob = 1;
          koff[t] = phys * ps[0] + g * ps[1] + (t % block_size) * ps[2];
        }
        if (oob) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        /* the k and v pools share one addressing, so koff serves both */
        attend_row(q, kpool, vpool, dtype, d, scale, b * qs[0] + h * qs[1], koff, koff, n, s,
                   o + r * d, lse + r);
      }
    }
    free(s);
    free(koff);
  }
  return bad;
}

/*
 * Paged (chunked) prefill: a chunk of new queries per sequence against that
 * sequence's whole context in a paged pool.  q is packed [Tq, Hq, d] (element
 * strides {token, head}); sequence s owns query tokens [cu_q[s], cu_q[s+1])
 * and seq_lens_k[s] logical keys, key t at
 * pool[block_table[s][t / block]][g][t % block] as in the paged decode
 * ("S12 FlashAttention", section "What this unlocks beyond speed": the tiles
 * of a sequence need not be contiguous).  Causal alignment as for dense
 * attention: query i of the chunk (0-based) sees key t iff
 * t <= i + (seq_lens_k[s] - chunk length).  Rows are flattened ids
 * r = h * Tq + t (rows == NULL: all Hq*Tq).
 */
int oracle_attn_paged_prefill(const void *q, const void *kpool, const void *vpool, int dtype,
                              const int32_t *cu_q, int nseq, const int64_t *qs, const int64_t *ps,
                              const int32_t *block_table, int max_blocks,
                              const int32_t *seq_lens_k, int Hq, int Hkv, int d, int block_size,
                              int num_blocks, int causal, double scale, const int64_t *rows,
                              int64_t nrows, double *o, double *lse, int nthreads) {
  if (!q || !cu_q || !qs || !ps || !block_table || !seq_lens_k || !o || !lse) return 1;
  if (nseq < 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || Hq % Hkv || block_size <= 0) return 1;
  if (cu_q[0] != 0) return 1;
  int64_t maxlen = 1;
  for (int s = 0; s < nseq; ++s) {
    if (cu_q[s + 1] < cu_q[s]) return 1;
    if (seq_lens_k[s] < 0 || (int64_t)seq_lens_k[s] > (int64_t)max_blocks * block_size) return 1;
    if (seq_lens_k[s] > maxlen) maxlen = seq_lens_k[s];
  }
  if (maxlen > 1 && (!kpool || !vpool)) return 1;
  const int64_t T = cu_q[nseq];
  if (!rows) nrows = (int64_t)Hq * T;
  const int group = Hq / Hkv;
  int bad = 0;
  set_threads(nthreads);
#pragma omp parallel
  {
    double *s = (double *)malloc(sizeof(double) * (size_t)maxlen);
    int64_t *koff = (int64_t *)malloc(sizeof(int64_t) * (size_t)maxlen);
    if (!s || !koff) {
#pragma omp atomic write
      bad = 2;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t r = 0; r < nrows; ++r) {
        int64_t id = rows ? rows[r] : r;
        int64_t t = id % (T > 0 ? T : 1), h = id / (T > 0 ? T : 1);
        if (id < 0 || h >= Hq || T == 0) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        int seq = 0;
        while (cu_q[seq + 1] <= t) ++seq; /* the sequence holding query token t */
        int64_t nq = cu_q[seq + 1] - cu_q[seq], nk = seq_lens_k[seq];
        int64_t i = t - cu_q[seq];
        int64_t n = causal ? i + 1 + (nk - nq) : nk; /* keys 0 .. n-1 are visible */
        if (n > nk) n = nk;
        if (n < 0) n = 0;
        int64_t g = h / group;
        int oob = 0;
        for (int64_t j = 0; j < n; ++j) {
          int64_t phys = block_table[seq * (int64_t)max_blocks + j / block_size];
          if (phys < 0 || phys >= num_blocks) oob = 1;
          koff[j] = phys * ps[0] + g * ps[1] + (j % block_size) * ps[2];
        }
        if (oob) {
#pragma omp atomic write
          bad = 1;
          continue;
        }
        /* the k and v pools share one addressing, so koff serves both */
        attend_row(q, kpool, vpool, dtype, d, scale, t * qs[0] + h * qs[1], koff, koff, n, s,
                   o + r * d, lse + r);
      }
    }
    free(s);
    free(koff);
  }
  return bad;
}

/*
 * Merge of P partial attention results of the same R query rows over
 * disjoint key sets ("FlashAttention", tachyon.techntrek.in, "For engineers /
 * Show the maths": two states (m, l, o) combine by rescaling both to the
 * larger max and adding; here all P states at once).  Part p gives its
 * normalised output o_p (d values per row) and lse_p = m_p + log l_p; against
 * m = max_p lse_p part p weighs w_p = exp(lse_p - m) = l_p exp(m_p - m), and
 * the union is o = sum_p w_p o_p / sum_p w_p, lse = m + log sum_p w_p.  A part
 * with lse_p = -inf saw no key for that row and is skipped (its o_p is not
 * read); a row no part saw gets o = 0, lse = -inf.
 * Layouts: o_parts [P][R][d], lse_parts [P][R], o [R][d], lse [R].
 */
void oracle_merge_states(int64_t P, int64_t R, int64_t d, const double *o_parts, const double *lse_parts,
                         double *o, double *lse) {
  for (int64_t r = 0; r < R; ++r) {
    double m = -INFINITY;
    for (int64_t p = 0; p < P; ++p)
      if (lse_parts[p * R + r] > m) m = lse_parts[p * R + r];
    double *orow = o + r * d;
    for (int64_t c = 0; c < d; ++c) orow[c] = 0.0;
    if (m == -INFINITY) {
      lse[r] = -INFINITY;
      continue;
    }
    double z = 0.0;
    for (int64_t p = 0; p < P; ++p) {
      const double lp = lse_parts[p * R + r];
      if (lp == -INFINITY) continue;
      const double w = exp(lp - m);
      z += w;
      for (int64_t c = 0; c < d; ++c) orow[c] += w * o_parts[(p * R + r) * d + c];
    }
    for (int64_t c = 0; c < d; ++c) orow[c] /= z;
    lse[r] = m + log(z);
  }
}
