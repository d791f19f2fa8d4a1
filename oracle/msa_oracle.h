/*
 * CPU oracle for top-k block-sparse GQA attention (forward) and its k2q CSR.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing on the product path may include, link,
 * load or call this code: only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg use it. It shares no code with the HIP
 * library. All pointers are host memory. bf16 tensors are passed as their
 * 16-bit patterns and widened exactly; all arithmetic is in double.
 *
 * Definitions follow the page "MiniMax-AI/MSA python/fmha_sm100/cute/
 * test_sparse_atten.py": the golden reference `sparse_attention_ref`
 * (block mask from the index table with set semantics, -1 ignored, GQA head
 * map by repeat-interleave, seqused_k mask, bottom-right causal limit
 * q + seqused_k - Sq, masked logsumexp in natural log, empty rows give
 * O = 0 and LSE = -inf), the paged packer `pack_paged_kv` (pool
 * [num_pages, Hkv, page_size, D] addressed through page_table[b][j / page])
 * and the page "MSA interface.py" (`sparse_atten_func`: default scale
 * D^-0.5; `build_k2q_csr`: kv-block -> query CSR, done once per call site).
 */
#ifndef MSA_ORACLE_H
#define MSA_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Sparse attention, contiguous K/V.
 *   q        [B, Sq, Hq, D]   bf16 bits
 *   k, v     [B, Skv, Hkv, D] bf16 bits, or fp8 e4m3fn bytes when kv_fp8 (the
 *            fp8 KV cache of `sparse_atten_func`: each K/V element is the
 *            e4m3fn value, used as is -- no scale)
 *   q2k      [B, Hkv, Sq, topk] int32 block ids, -1 (or any id outside
 *            [0, Skv/blk)) = unused slot; duplicates count once
 *   seqused_k NULL or [B]: keys j >= seqused_k[b] are masked and the causal
 *            limit uses seqused_k[b] in place of Skv
 *   rows     NULL (all B*Sq rows, in order) or nrows global row ids b*Sq+q
 *   o        [nrows, Hq, D] double;  lse [nrows, Hq] double (natural log)
 *   temp, lse_t  lse_t NULL, or [nrows, Hq]: the temperature-scaled LSE, the
 *            log-sum-exp of the same masked scores divided by temp > 0
 *            (`lse_temperature_scale` of `sparse_attention_ref` on the test
 *            page and of `sparse_atten_func` on the interface page)
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_sparse_attention(const uint16_t* q, const void* k, const void* v, int kv_fp8,
                            const int32_t* q2k, const int32_t* seqused_k, int B, int Sq, int Skv,
                            int Hq, int Hkv, int D, int topk, int blk, int causal, double scale,
                            const int64_t* rows, int64_t nrows, double* o, double* lse,
                            double temp, double* lse_t, int nthreads);

/*
 * Sparse attention, paged K/V. Logical block s of sequence b is physical page
 * page_table[b * max_pages + s] (page_size == block size); a page id outside
 * [0, num_pages) makes that block contribute nothing. Keys j >= seqused_k[b]
 * are masked and the causal limit is q + seqused_k[b] - Sq. Valid block ids
 * are [0, max_pages). Other arguments as above.
 */
int oracle_paged_sparse_attention(const uint16_t* q, const void* k_pool, const void* v_pool,
                                  int kv_fp8, const int32_t* page_table,
                                  const int32_t* seqused_k, const int32_t* q2k, int B, int Sq,
                                  int Hq, int Hkv, int D, int topk, int page_size, int num_pages,
                                  int max_pages, int causal, double scale, const int64_t* rows,
                                  int64_t nrows, double* o, double* lse, double temp,
                                  double* lse_t, int nthreads);

/*
 * kv-block -> query CSR of a [B, Hkv, Sq, topk] index table.
 * Rows r = b * nblk + s per KV head. row_ptr [Hkv, B*nblk + 1];
 * q_idx and slot [Hkv, B*Sq*topk]: row r lists the global query ids b*Sq+q
 * whose row holds s, ascending in q then slot t, and slot[] holds that t.
 * Entries beyond row_ptr[h][B*nblk] are left untouched. slot may be NULL.
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_k2q_csr(const int32_t* q2k, int B, int Hkv, int Sq, int topk, int nblk,
                   int32_t* row_ptr, int32_t* q_idx, int32_t* slot);

/*
 * Variable-length batches (the packed form of `sparse_atten_func` on the page
 * "MSA interface.py": cu_seqlens_q / cu_seqlens_k prefix sums, q2k
 * [Hkv, total_q, topK]). Sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and
 * keys cu_k[b] .. cu_k[b+1]-1; its block ids s count from its first key
 * (keys 128 s .. 128 s + 127 of the sequence, those >= its length masked),
 * valid ids are [0, ceil(Skv_b / blk)), and the causal limit is
 * q + Skv_b - Sq_b with q the row's position in its sequence. Each sequence is
 * the batched definition above with B = 1 (the page's varlen tests compare each
 * sequence against `sparse_attention_ref` that way).
 *   q     [total_q, Hq, D]; k, v [total_k, Hkv, D]; q2k [Hkv, total_q, topk]
 *   rows  NULL (all total_q rows) or nrows global row ids
 *   o     [nrows, Hq, D] double; lse [nrows, Hq] double
 */
int oracle_sparse_attention_varlen(const uint16_t* q, const void* k, const void* v, int kv_fp8,
                                   const int32_t* q2k, const int32_t* cu_seqlens_q,
                                   const int32_t* cu_seqlens_k, int B, int Hq, int Hkv, int D,
                                   int topk, int blk, int causal, double scale,
                                   const int64_t* rows, int64_t nrows, double* o, double* lse,
                                   double temp, double* lse_t, int nthreads);

/*
 * k2q CSR of a variable-length batch (`build_k2q_csr` with cu_seqlens and
 * total_rows on the page "MSA interface.py"): row r = rowbase[b] + s with
 * rowbase[b] = sum over b' < b of ceil(Skv_b' / blk); total_rows must equal
 * rowbase[B]. Entries of a row are global query ids g ascending, then slot t.
 *   row_ptr [Hkv, total_rows + 1]; q_idx, slot [Hkv, total_q * topk]
 */
int oracle_k2q_csr_varlen(const int32_t* q2k, const int32_t* cu_seqlens_q,
                          const int32_t* cu_seqlens_k, int B, int Hkv, int topk, int blk,
                          int total_rows, int32_t* row_ptr, int32_t* q_idx, int32_t* slot);

/*
 * The fp8 e4m3fn decoding the K/V reads use: n bytes -> n values (NaN for the
 * two NaN patterns). Returns 0, or -1 on invalid arguments.
 */
int oracle_fp8_e4m3_decode(const uint8_t* in, int64_t n, double* out);

/*
 * Rounding to the nearest fp8 e4m3fn value, ties to the even code (the
 * `.to(torch.float8_e4m3fn)` cast the test page applies to the unnormalised
 * probabilities of the fp8 decode): n values -> n values. Finite magnitudes up
 * to 448 round into the format (subnormal step 2^-9, 3 mantissa bits above
 * 2^-6); magnitudes >= 464 and NaN give NaN (the format has no infinity).
 * Returns 0, or -1 on invalid arguments.
 */
int oracle_fp8_e4m3_round(const double* in, int64_t n, double* out);

/*
 * The fp8 dense paged decode of the test page (`_decode_paged_dense_reference`,
 * checked against `sparse_decode_atten_func` with q2k = None): Q, K and V are
 * fp8 e4m3fn bytes; every key of the sequence is visible up to seqused_k[b]
 * (and the bottom-right causal limit q + seqused_k[b] - Sq when causal). Per
 * (row, head), with scores s_j = scale * q . k_j and m = max_j s_j:
 *   row_sum = sum_j exp(s_j - m)                      (unrounded)
 *   O       = sum_j e4m3(exp(s_j - m)) v_j / row_sum  (probabilities rounded
 *                                                      to e4m3 before P V)
 *   LSE     = m + log(row_sum)
 * Empty rows give O = 0, LSE = -inf. A page id outside [0, num_pages) makes its
 * keys contribute nothing.
 *   q        [B * Sq, Hq, D] fp8 bytes
 *   k_pool, v_pool  [num_pages, Hkv, page_size, D] fp8 bytes
 *   page_table [B, max_pages]; seqused_k [B]
 *   rows, o, lse, temp, lse_t  as for oracle_paged_sparse_attention (lse_t is the
 *            log-sum-exp of the unrounded scores divided by temp)
 */
int oracle_paged_decode_fp8(const uint8_t* q, const uint8_t* k_pool, const uint8_t* v_pool,
                            const int32_t* page_table, const int32_t* seqused_k, int B, int Sq,
                            int Hq, int Hkv, int D, int page_size, int num_pages, int max_pages,
                            int causal, double scale, const int64_t* rows, int64_t nrows,
                            double* o, double* lse, double temp, double* lse_t, int nthreads);

#ifdef __cplusplus
}
#endif
#endif
