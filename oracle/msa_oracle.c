/*
 * CPU oracle for top-k block-sparse GQA attention (forward) and its k2q CSR.
 *
 * TEST INFRASTRUCTURE ONLY: used by the test suite, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. Plain loops in
 * double precision, one query row at a time; the only parallelism is an
 * OpenMP loop over independent query rows. The definitions it writes out are
 * cited in msa_oracle.h.
 */
#include "msa_oracle.h"

#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* fp8 e4m3fn (1 sign, 4 exponent bits with bias 7, 3 mantissa bits; no infinities;
 * exponent and mantissa all ones = NaN): (-1)^s (1 + m/8) 2^(e-7), or m 2^-9 for e = 0 */
static double fp8_value(uint8_t bits) {
  const int s = bits >> 7, e = (bits >> 3) & 15, m = bits & 7;
  if (e == 15 && m == 7) return NAN;
  const double v = e == 0 ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

int oracle_fp8_e4m3_decode(const uint8_t* in, int64_t n, double* out) {
  if (!in || !out || n < 0) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = fp8_value(in[i]);
  return 0;
}

/* Where the keys and values of one sequence live. */
typedef struct {
  const void* k;  /* bf16 bits, or fp8 e4m3fn bytes when fp8 */
  const void* v;
  const int32_t* page_table; /* NULL: contiguous [B, Skv, Hkv, D] */
  int Skv;                   /* contiguous only */
  int Hkv, D, page_size, num_pages, max_pages;
  int fp8;                   /* K/V stored as fp8 e4m3fn */
} kv_source;

static double k_value(const kv_source* s, int64_t i) {
  return s->fp8 ? fp8_value(((const uint8_t*)s->k)[i]) : bf16_value(((const uint16_t*)s->k)[i]);
}
static double v_value(const kv_source* s, int64_t i) {
  return s->fp8 ? fp8_value(((const uint8_t*)s->v)[i]) : bf16_value(((const uint16_t*)s->v)[i]);
}

/* Row offset (in elements) of key/value token j of sequence b, head hkv,
 * or -1 when the token has no storage (page id out of range). */
static int64_t kv_offset(const kv_source* s, int b, int hkv, int64_t j) {
  if (!s->page_table) return (((int64_t)b * s->Skv + j) * s->Hkv + hkv) * s->D;
  int64_t page = s->page_table[(int64_t)b * s->max_pages + j / s->page_size];
  if (page < 0 || page >= s->num_pages) return -1;
  return ((page * s->Hkv + hkv) * s->page_size + j % s->page_size) * s->D;
}

/*
 * One query row: all Hq heads.
 *   qrow       the row's Q, [Hq, D]
 *   sel0       the row's index slots for KV head 0; KV head hkv's slots are at
 *              sel0 + hkv * sel_stride
 *   b          the sequence (K/V source coordinate)
 *   qpos, Sq   position of the row in its sequence and the sequence's length
 *   nblk       valid block ids are [0, nblk)
 *   kvlen      keys j >= kvlen are masked
 *   temp, lset_row  when lset_row is not NULL it receives, per head, the log-sum-exp
 *              of the same masked scores divided by temp (the temperature-scaled LSE)
 *   The causal limit is qpos + kvlen - Sq (bottom-right alignment).
 */
static void attend_row(const kv_source* src, const uint16_t* qrow, const int32_t* sel0,
                       int64_t sel_stride, int b, int qpos, int Sq, int Hq, int Hkv, int D,
                       int topk, int blk, int nblk, int64_t kvlen, int causal, double scale,
                       unsigned char* mark, double* score, double* acc, double* o_row,
                       double* lse_row, double temp, double* lset_row) {
  const int qpk = Hq / Hkv;
  const int64_t limit = causal ? (int64_t)qpos + kvlen - Sq : INT64_MAX;
  for (int hkv = 0; hkv < Hkv; ++hkv) {
    /* selected set: each valid block id once */
    if (nblk > 0) memset(mark, 0, (size_t)nblk);
    const int32_t* sel = sel0 + hkv * sel_stride;
    for (int t = 0; t < topk; ++t)
      if (sel[t] >= 0 && sel[t] < nblk) mark[sel[t]] = 1;

    for (int h = hkv * qpk; h < (hkv + 1) * qpk; ++h) {
      const uint16_t* qh = qrow + (int64_t)h * D;
      double* oh = o_row + (int64_t)h * D;
      /* scores of the visible keys, in ascending key order */
      int64_t n = 0;
      double m = -INFINITY;
      for (int s = 0; s < nblk; ++s) {
        if (!mark[s]) continue;
        for (int r = 0; r < blk; ++r) {
          const int64_t j = (int64_t)s * blk + r;
          if (j >= kvlen || j > limit) continue;
          const int64_t off = kv_offset(src, b, hkv, j);
          if (off < 0) continue;
          double dot = 0.0;
          for (int d = 0; d < D; ++d) dot += bf16_value(qh[d]) * k_value(src, off + d);
          score[n++] = scale * dot;
          if (scale * dot > m) m = scale * dot;
        }
      }
      if (n == 0) {
        for (int d = 0; d < D; ++d) oh[d] = 0.0;
        lse_row[h] = -INFINITY;
        if (lset_row) lset_row[h] = -INFINITY;
        continue;
      }
      /* log sum_j exp(s_j / temp) = m / temp + log sum_j exp((s_j - m) / temp), temp > 0 */
      if (lset_row) {
        double lt = 0.0;
        for (int64_t i2 = 0; i2 < n; ++i2) lt += exp((score[i2] - m) / temp);
        lset_row[h] = m / temp + log(lt);
      }
      /* softmax-weighted sum of the values, same key order */
      for (int d = 0; d < D; ++d) acc[d] = 0.0;
      double l = 0.0;
      int64_t i = 0;
      for (int s = 0; s < nblk; ++s) {
        if (!mark[s]) continue;
        for (int r = 0; r < blk; ++r) {
          const int64_t j = (int64_t)s * blk + r;
          if (j >= kvlen || j > limit) continue;
          const int64_t off = kv_offset(src, b, hkv, j);
          if (off < 0) continue;
          const double p = exp(score[i++] - m);
          l += p;
          for (int d = 0; d < D; ++d) acc[d] += p * v_value(src, off + d);
        }
      }
      for (int d = 0; d < D; ++d) oh[d] = acc[d] / l;
      lse_row[h] = m + log(l);
    }
  }
}

static int run_rows(const kv_source* src, const uint16_t* q, const int32_t* q2k,
                    const int32_t* seqused_k, int B, int Sq, int Hq, int Hkv, int D, int topk,
                    int blk, int nblk, int64_t full_len, int causal, double scale,
                    const int64_t* rows, int64_t nrows, double* o, double* lse, double temp,
                    double* lse_t, int nthreads) {
  if (!rows) nrows = (int64_t)B * Sq;
  int failed = 0;
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    unsigned char* mark = (unsigned char*)malloc((size_t)(nblk > 0 ? nblk : 1));
    double* score = (double*)malloc(sizeof(double) * (size_t)topk * (size_t)blk);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!mark || !score || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t i = 0; i < nrows; ++i) {
        const int64_t g = rows ? rows[i] : i;
        if (g < 0 || g >= (int64_t)B * Sq) {
#pragma omp atomic write
          failed = 1;
          continue;
        }
        const int b = (int)(g / Sq), qpos = (int)(g % Sq);
        int64_t kvlen = full_len;
        if (seqused_k && seqused_k[b] < kvlen) kvlen = seqused_k[b];
        if (kvlen < 0) kvlen = 0;
        attend_row(src, q + g * Hq * D, q2k + (((int64_t)b * Hkv) * Sq + qpos) * topk,
                   (int64_t)Sq * topk, b, qpos, Sq, Hq, Hkv, D, topk, blk, nblk, kvlen, causal,
                   scale, mark, score, acc, o + i * Hq * D, lse + i * Hq, temp,
                   lse_t ? lse_t + i * Hq : NULL);
      }
    }
    free(mark);
    free(score);
    free(acc);
  }
  return failed ? -1 : 0;
}

int oracle_sparse_attention(const uint16_t* q, const void* k, const void* v, int kv_fp8,
                            const int32_t* q2k, const int32_t* seqused_k, int B, int Sq, int Skv,
                            int Hq, int Hkv, int D, int topk, int blk, int causal, double scale,
                            const int64_t* rows, int64_t nrows, double* o, double* lse,
                            double temp, double* lse_t, int nthreads) {
  if (!q || !k || !v || !q2k || !o || !lse || B <= 0 || Sq <= 0 || Skv <= 0 || Hkv <= 0 ||
      Hq <= 0 || Hq % Hkv || D <= 0 || topk <= 0 || blk <= 0 || Skv % blk ||
      (lse_t && !(temp > 0.0)))
    return -1;
  kv_source src = {k, v, NULL, Skv, Hkv, D, blk, 0, 0, kv_fp8 ? 1 : 0};
  return run_rows(&src, q, q2k, seqused_k, B, Sq, Hq, Hkv, D, topk, blk, Skv / blk, Skv, causal,
                  scale, rows, nrows, o, lse, temp, lse_t, nthreads);
}

int oracle_paged_sparse_attention(const uint16_t* q, const void* k_pool, const void* v_pool,
                                  int kv_fp8, const int32_t* page_table,
                                  const int32_t* seqused_k, const int32_t* q2k, int B, int Sq,
                                  int Hq, int Hkv, int D, int topk, int page_size, int num_pages,
                                  int max_pages, int causal, double scale, const int64_t* rows,
                                  int64_t nrows, double* o, double* lse, double temp,
                                  double* lse_t, int nthreads) {
  if (!q || !k_pool || !v_pool || !page_table || !seqused_k || !q2k || !o || !lse || B <= 0 ||
      Sq <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || D <= 0 || topk <= 0 || page_size <= 0 ||
      num_pages <= 0 || max_pages <= 0 || (lse_t && !(temp > 0.0)))
    return -1;
  kv_source src = {k_pool, v_pool, page_table, 0, Hkv, D, page_size, num_pages, max_pages,
                   kv_fp8 ? 1 : 0};
  return run_rows(&src, q, q2k, seqused_k, B, Sq, Hq, Hkv, D, topk, page_size, max_pages,
                  (int64_t)max_pages * page_size, causal, scale, rows, nrows, o, lse, temp,
                  lse_t, nthreads);
}

int oracle_k2q_csr(const int32_t* q2k, int B, int Hkv, int Sq, int topk, int nblk,
                   int32_t* row_ptr, int32_t* q_idx, int32_t* slot) {
  if (!q2k || !row_ptr || !q_idx || B <= 0 || Hkv <= 0 || Sq <= 0 || topk <= 0 || nblk <= 0)
    return -1;
  const int64_t nrows = (int64_t)B * nblk;
  const int64_t cap = (int64_t)B * Sq * topk;
  int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)nrows);
  if (!cursor) return -1;
  for (int hkv = 0; hkv < Hkv; ++hkv) {
    int32_t* rp = row_ptr + hkv * (nrows + 1);
    /* count the valid (q, t) entries of each row */
    for (int64_t r = 0; r <= nrows; ++r) rp[r] = 0;
    for (int b = 0; b < B; ++b)
      for (int qpos = 0; qpos < Sq; ++qpos) {
        const int32_t* sel = q2k + (((int64_t)b * Hkv + hkv) * Sq + qpos) * topk;
        for (int t = 0; t < topk; ++t)
          if (sel[t] >= 0 && sel[t] < nblk) rp[(int64_t)b * nblk + sel[t] + 1] += 1;
      }
    /* exclusive prefix sum */
    for (int64_t r = 0; r < nrows; ++r) rp[r + 1] += rp[r];
    /* place entries in ascending (q, t) order */
    for (int64_t r = 0; r < nrows; ++r) cursor[r] = rp[r];
    for (int b = 0; b < B; ++b)
      for (int qpos = 0; qpos < Sq; ++qpos) {
        const int32_t* sel = q2k + (((int64_t)b * Hkv + hkv) * Sq + qpos) * topk;
        for (int t = 0; t < topk; ++t) {
          if (sel[t] < 0 || sel[t] >= nblk) continue;
          const int64_t pos = cursor[(int64_t)b * nblk + sel[t]]++;
          q_idx[hkv * cap + pos] = (int32_t)((int64_t)b * Sq + qpos);
          if (slot) slot[hkv * cap + pos] = t;
        }
      }
  }
  free(cursor);
  return 0;
}

/* Sequence of global query row g: the b with cu_q[b] <= g < cu_q[b + 1]. */
static int sequence_of(const int32_t* cu_q, int B, int64_t g) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) / 2;
    if (cu_q[mid] <= g) lo = mid; else hi = mid - 1;
  }
  return lo;
}

static int varlen_args_ok(const int32_t* cu_q, const int32_t* cu_k, int B) {
  if (!cu_q || !cu_k || B <= 0 || cu_q[0] != 0 || cu_k[0] != 0) return 0;
  for (int b = 0; b < B; ++b)
    if (cu_q[b + 1] < cu_q[b] || cu_k[b + 1] < cu_k[b]) return 0;
  return 1;
}

int oracle_sparse_attention_varlen(const uint16_t* q, const void* k, const void* v, int kv_fp8,
                                   const int32_t* q2k, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int D,
                                   int topk, int blk, int causal, double scale,
                                   const int64_t* rows, int64_t nrows, double* o, double* lse,
                                   double temp, double* lse_t, int nthreads) {
  if (!q || !k || !v || !q2k || !o || !lse || Hkv <= 0 || Hq <= 0 || Hq % Hkv || D <= 0 ||
      topk <= 0 || blk <= 0 || !varlen_args_ok(cu_seqlens_q, cu_seqlens_k, B) ||
      (lse_t && !(temp > 0.0)))
    return -1;
  const int64_t total_q = cu_seqlens_q[B];
  int max_nblk = 1;
  for (int b = 0; b < B; ++b) {
    const int nb = (cu_seqlens_k[b + 1] - cu_seqlens_k[b] + blk - 1) / blk;
    if (nb > max_nblk) max_nblk = nb;
  }
  if (!rows) nrows = total_q;
  int failed = 0;
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    unsigned char* mark = (unsigned char*)malloc((size_t)max_nblk);
    double* score = (double*)malloc(sizeof(double) * (size_t)topk * (size_t)blk);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!mark || !score || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 4)
      for (int64_t i = 0; i < nrows; ++i) {
        const int64_t g = rows ? rows[i] : i;
        if (g < 0 || g >= total_q) {
#pragma omp atomic write
          failed = 1;
          continue;
        }
        /* the row's sequence: its keys are tokens cu_k[b] .. cu_k[b+1]-1 of k/v, its
         * block ids count from that sequence's first token */
        const int b = sequence_of(cu_seqlens_q, B, g);
        const int Sq_b = cu_seqlens_q[b + 1] - cu_seqlens_q[b];
        const int Skv_b = cu_seqlens_k[b + 1] - cu_seqlens_k[b];
        const int nblk_b = (Skv_b + blk - 1) / blk;
        const int64_t koff = (int64_t)cu_seqlens_k[b] * Hkv * D * (kv_fp8 ? 1 : 2);
        const kv_source src = {(const char*)k + koff, (const char*)v + koff, NULL, Skv_b, Hkv,
                               D, blk, 0, 0, kv_fp8 ? 1 : 0};
        attend_row(&src, q + g * Hq * D, q2k + g * topk, total_q * topk, 0,
                   (int)(g - cu_seqlens_q[b]), Sq_b, Hq, Hkv, D, topk, blk, nblk_b, Skv_b,
                   causal, scale, mark, score, acc, o + i * Hq * D, lse + i * Hq, temp,
                   lse_t ? lse_t + i * Hq : NULL);
      }
    }
    free(mark);
    free(score);
    free(acc);
  }
  return failed ? -1 : 0;
}

int oracle_k2q_csr_varlen(const int32_t* q2k, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int B, int Hkv, int topk, int blk,
                          int total_rows, int32_t* row_ptr, int32_t* q_idx, int32_t* slot) {
  if (!q2k || !row_ptr || !q_idx || Hkv <= 0 || topk <= 0 || blk <= 0 ||
      !varlen_args_ok(cu_seqlens_q, cu_seqlens_k, B))
    return -1;
  /* row r = rowbase[b] + s for block s of sequence b */
  int64_t* rowbase = (int64_t*)malloc(sizeof(int64_t) * (size_t)(B + 1));
  if (!rowbase) return -1;
  rowbase[0] = 0;
  for (int b = 0; b < B; ++b)
    rowbase[b + 1] = rowbase[b] + (cu_seqlens_k[b + 1] - cu_seqlens_k[b] + blk - 1) / blk;
  if (rowbase[B] != total_rows) {
    free(rowbase);
    return -1;
  }
  const int64_t total_q = cu_seqlens_q[B];
  const int64_t cap = total_q * topk;
  int64_t* cursor = (int64_t*)malloc(sizeof(int64_t) * (size_t)(total_rows > 0 ? total_rows : 1));
  if (!cursor) {
    free(rowbase);
    return -1;
  }
  for (int hkv = 0; hkv < Hkv; ++hkv) {
    int32_t* rp = row_ptr + (int64_t)hkv * (total_rows + 1);
    for (int64_t r = 0; r <= total_rows; ++r) rp[r] = 0;
    /* count, then place in ascending (global query, slot) order */
    for (int pass = 0; pass < 2; ++pass) {
      if (pass == 1) {
        for (int64_t r = 0; r < total_rows; ++r) rp[r + 1] += rp[r];
        for (int64_t r = 0; r < total_rows; ++r) cursor[r] = rp[r];
      }
      for (int b = 0; b < B; ++b) {
        const int nblk_b = (int)(rowbase[b + 1] - rowbase[b]);
        for (int64_t g = cu_seqlens_q[b]; g < cu_seqlens_q[b + 1]; ++g) {
          const int32_t* sel = q2k + ((int64_t)hkv * total_q + g) * topk;
          for (int t = 0; t < topk; ++t) {
            if (sel[t] < 0 || sel[t] >= nblk_b) continue;
            const int64_t r = rowbase[b] + sel[t];
            if (pass == 0) {
              rp[r + 1] += 1;
            } else {
              const int64_t pos = cursor[r]++;
              q_idx[hkv * cap + pos] = (int32_t)g;
              if (slot) slot[hkv * cap + pos] = t;
            }
          }
        }
      }
    }
  }
  free(cursor);
  free(rowbase);
  return 0;
}

/* Nearest fp8 e4m3fn value of x, ties to the even code: 4 significant bits for
 * |x| >= 2^-6 (quantum 2^(e-4) with |x| = f 2^e, f in [0.5, 1)), a fixed
 * quantum of 2^-9 below; rint rounds half to even in the default mode. */
static double fp8_round(double x) {
  if (isnan(x)) return NAN;
  const double a = fabs(x);
  if (a >= 464.0) return NAN;  /* past the midpoint above 448: no finite code */
  double r;
  if (a < ldexp(1.0, -6)) {
    r = ldexp(rint(ldexp(a, 9)), -9);
  } else {
    int e;
    frexp(a, &e);
    r = ldexp(rint(ldexp(a, 4 - e)), e - 4);
    if (r > 448.0) r = 448.0;  /* (448, 464) rounds down to the largest code */
  }
  return x < 0 ? -r : r;
}

int oracle_fp8_e4m3_round(const double* in, int64_t n, double* out) {
  if (!in || !out || n < 0) return -1;
  for (int64_t i = 0; i < n; ++i) out[i] = fp8_round(in[i]);
  return 0;
}

int oracle_paged_decode_fp8(const uint8_t* q, const uint8_t* k_pool, const uint8_t* v_pool,
                            const int32_t* page_table, const int32_t* seqused_k, int B, int Sq,
                            int Hq, int Hkv, int D, int page_size, int num_pages, int max_pages,
                            int causal, double scale, const int64_t* rows, int64_t nrows,
                            double* o, double* lse, double temp, double* lse_t, int nthreads) {
  if (!q || !k_pool || !v_pool || !page_table || !seqused_k || !o || !lse || B <= 0 || Sq <= 0 ||
      Hkv <= 0 || Hq <= 0 || Hq % Hkv || D <= 0 || page_size <= 0 || num_pages <= 0 ||
      max_pages <= 0 || (lse_t && !(temp > 0.0)))
    return -1;
  if (!rows) nrows = (int64_t)B * Sq;
  const int qpk = Hq / Hkv;
  const int64_t full_len = (int64_t)max_pages * page_size;
  kv_source src = {k_pool, v_pool, page_table, 0, Hkv, D, page_size, num_pages, max_pages, 1};
  int failed = 0;
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    double* score = (double*)malloc(sizeof(double) * (size_t)(full_len > 0 ? full_len : 1));
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!score || !acc) {
#pragma omp atomic write
      failed = 1;
    } else {
#pragma omp for schedule(dynamic, 1)
      for (int64_t i = 0; i < nrows; ++i) {
        const int64_t g = rows ? rows[i] : i;
        if (g < 0 || g >= (int64_t)B * Sq) {
#pragma omp atomic write
          failed = 1;
          continue;
        }
        const int b = (int)(g / Sq), qpos = (int)(g % Sq);
        int64_t kvlen = seqused_k[b] < full_len ? seqused_k[b] : full_len;
        if (kvlen < 0) kvlen = 0;
        const int64_t limit = causal ? (int64_t)qpos + kvlen - Sq : INT64_MAX;
        for (int h = 0; h < Hq; ++h) {
          const int hkv = h / qpk;
          const uint8_t* qh = q + (g * Hq + h) * D;
          double* oh = o + (i * Hq + h) * D;
          /* pass 1: scores of the visible keys (ascending key order) and their max */
          int64_t n = 0;
          double m = -INFINITY;
          for (int64_t j = 0; j < kvlen && j <= limit; ++j) {
            const int64_t off = kv_offset(&src, b, hkv, j);
            if (off < 0) continue;
            double dot = 0.0;
            for (int d = 0; d < D; ++d) dot += fp8_value(qh[d]) * k_value(&src, off + d);
            score[n++] = scale * dot;
            if (scale * dot > m) m = scale * dot;
          }
          if (n == 0) {
            for (int d = 0; d < D; ++d) oh[d] = 0.0;
            lse[i * Hq + h] = -INFINITY;
            if (lse_t) lse_t[i * Hq + h] = -INFINITY;
            continue;
          }
          if (lse_t) {
            double lt = 0.0;
            for (int64_t k2 = 0; k2 < n; ++k2) lt += exp((score[k2] - m) / temp);
            lse_t[i * Hq + h] = m / temp + log(lt);
          }
          /* pass 2: unrounded row sum; values weighted by the e4m3-rounded probabilities */
          for (int d = 0; d < D; ++d) acc[d] = 0.0;
          double l = 0.0;
          int64_t k1 = 0;
          for (int64_t j = 0; j < kvlen && j <= limit; ++j) {
            const int64_t off = kv_offset(&src, b, hkv, j);
            if (off < 0) continue;
            const double p = exp(score[k1++] - m);
            l += p;
            const double pq = fp8_round(p);
            for (int d = 0; d < D; ++d) acc[d] += pq * v_value(&src, off + d);
          }
          for (int d = 0; d < D; ++d) oh[d] = acc[d] / l;
          lse[i * Hq + h] = m + log(l);
        }
      }
    }
    free(score);
    free(acc);
  }
  return failed ? -1 : 0;
}
