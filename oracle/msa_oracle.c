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

/* Where the keys and values of one sequence live. */
typedef struct {
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* page_table; /* NULL: contiguous [B, Skv, Hkv, D] */
  int Skv;                   /* contiguous only */
  int Hkv, D, page_size, num_pages, max_pages;
} kv_source;

/* Row offset (in elements) of key/value token j of sequence b, head hkv,
 * or -1 when the token has no storage (page id out of range). */
static int64_t kv_offset(const kv_source* s, int b, int hkv, int64_t j) {
  if (!s->page_table) return (((int64_t)b * s->Skv + j) * s->Hkv + hkv) * s->D;
  int64_t page = s->page_table[(int64_t)b * s->max_pages + j / s->page_size];
  if (page < 0 || page >= s->num_pages) return -1;
  return ((page * s->Hkv + hkv) * s->page_size + j % s->page_size) * s->D;
}

/*
 * One query row (b, qpos): all Hq heads.
 *   nblk   valid block ids are [0, nblk)
 *   kvlen  keys j >= kvlen are masked
 *   The causal limit is qpos + kvlen - Sq (bottom-right alignment).
 */
static void attend_row(const kv_source* src, const uint16_t* q, const int32_t* q2k, int b, int qpos,
                       int Sq, int Hq, int Hkv, int D, int topk, int blk, int nblk, int64_t kvlen,
                       int causal, double scale, unsigned char* mark, double* score, double* acc,
                       double* o_row, double* lse_row) {
  const int qpk = Hq / Hkv;
  const int64_t limit = causal ? (int64_t)qpos + kvlen - Sq : INT64_MAX;
  for (int hkv = 0; hkv < Hkv; ++hkv) {
    /* selected set: each valid block id once */
    memset(mark, 0, (size_t)nblk);
    const int32_t* sel = q2k + (((int64_t)b * Hkv + hkv) * Sq + qpos) * topk;
    for (int t = 0; t < topk; ++t)
      if (sel[t] >= 0 && sel[t] < nblk) mark[sel[t]] = 1;

    for (int h = hkv * qpk; h < (hkv + 1) * qpk; ++h) {
      const uint16_t* qh = q + (((int64_t)b * Sq + qpos) * Hq + h) * D;
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
          for (int d = 0; d < D; ++d) dot += bf16_value(qh[d]) * bf16_value(src->k[off + d]);
          score[n++] = scale * dot;
          if (scale * dot > m) m = scale * dot;
        }
      }
      if (n == 0) {
        for (int d = 0; d < D; ++d) oh[d] = 0.0;
        lse_row[h] = -INFINITY;
        continue;
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
          for (int d = 0; d < D; ++d) acc[d] += p * bf16_value(src->v[off + d]);
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
                    const int64_t* rows, int64_t nrows, double* o, double* lse, int nthreads) {
  if (!rows) nrows = (int64_t)B * Sq;
  int failed = 0;
  const int nt = nthreads > 0 ? nthreads : omp_get_max_threads();
#pragma omp parallel num_threads(nt)
  {
    unsigned char* mark = (unsigned char*)malloc((size_t)nblk);
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
        attend_row(src, q, q2k, b, qpos, Sq, Hq, Hkv, D, topk, blk, nblk, kvlen, causal, scale,
                   mark, score, acc, o + i * Hq * D, lse + i * Hq);
      }
    }
    free(mark);
    free(score);
    free(acc);
  }
  return failed ? -1 : 0;
}

int oracle_sparse_attention(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                            const int32_t* q2k, const int32_t* seqused_k, int B, int Sq, int Skv,
                            int Hq, int Hkv, int D, int topk, int blk, int causal, double scale,
                            const int64_t* rows, int64_t nrows, double* o, double* lse,
                            int nthreads) {
  if (!q || !k || !v || !q2k || !o || !lse || B <= 0 || Sq <= 0 || Skv <= 0 || Hkv <= 0 ||
      Hq <= 0 || Hq % Hkv || D <= 0 || topk <= 0 || blk <= 0 || Skv % blk)
    return -1;
  kv_source src = {k, v, NULL, Skv, Hkv, D, blk, 0, 0};
  return run_rows(&src, q, q2k, seqused_k, B, Sq, Hq, Hkv, D, topk, blk, Skv / blk, Skv, causal,
                  scale, rows, nrows, o, lse, nthreads);
}

int oracle_paged_sparse_attention(const uint16_t* q, const uint16_t* k_pool,
                                  const uint16_t* v_pool, const int32_t* page_table,
                                  const int32_t* seqused_k, const int32_t* q2k, int B, int Sq,
                                  int Hq, int Hkv, int D, int topk, int page_size, int num_pages,
                                  int max_pages, int causal, double scale, const int64_t* rows,
                                  int64_t nrows, double* o, double* lse, int nthreads) {
  if (!q || !k_pool || !v_pool || !page_table || !seqused_k || !q2k || !o || !lse || B <= 0 ||
      Sq <= 0 || Hkv <= 0 || Hq <= 0 || Hq % Hkv || D <= 0 || topk <= 0 || page_size <= 0 ||
      num_pages <= 0 || max_pages <= 0)
    return -1;
  kv_source src = {k_pool, v_pool, page_table, 0, Hkv, D, page_size, num_pages, max_pages};
  return run_rows(&src, q, q2k, seqused_k, B, Sq, Hq, Hkv, D, topk, page_size, max_pages,
                  (int64_t)max_pages * page_size, causal, scale, rows, nrows, o, lse, nthreads);
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
