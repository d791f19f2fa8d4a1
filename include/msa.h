/*
 * msa.h -- C ABI of the MI355X (gfx950) top-k block-sparse GQA attention library.
 *
 * The operation is the forward pass of the sparse attention defined on the
 * page "MiniMax-AI/MSA python/fmha_sm100/cute/test_sparse_atten.py"
 * (golden reference `sparse_attention_ref`) and exposed on the page
 * "MSA interface.py" (`sparse_atten_func`, `build_k2q_csr`,
 * `sparse_decode_atten_func`). For query row q of sequence b and query head
 * h (KV head hkv = h / (Hq / Hkv), the repeat-interleave GQA map):
 *
 *   selected  S = { q2k[b][hkv][q][t] : 0 <= value < nblk }   (a set; -1 = unused)
 *   keys      J = { j = blk*s + r : s in S, r < blk, j < kvlen_b,
 *                   and, if causal, j <= q + kvlen_b - Sq }      (bottom-right)
 *   O[b][q][h]   = sum_j softmax_j(scale * <Q, K_j>) V_j        (bf16 out)
 *   LSE[b][h][q] = log sum_j exp(scale * <Q, K_j>)               (natural log, fp32)
 *   J empty  ->  O = 0, LSE = -inf.
 *   Optionally the temperature-scaled LSE (lse_temperature_scale of
 *   sparse_atten_func): LSE_T[b][h][q] = log sum_j exp(scale * <Q, K_j> / T),
 *   -inf when J is empty.
 *
 * Conventions shared by every entry point
 *   - Device pointers unless stated. bf16 tensors are raw 16-bit patterns.
 *     Every tensor is dense row-major in the stated shape, 16-byte aligned.
 *   - The caller owns all memory and the stream. The library never allocates
 *     device memory, never synchronises the stream and keeps no state
 *     between calls beyond the thread-local error text and the optional
 *     profiling events of msa_set_profiling_events; calls are asynchronous on
 *     `stream` (a hipStream_t, NULL = the default stream).
 *   - Inputs are read only; outputs are fully overwritten; workspaces are
 *     scratch whose contents on entry do not matter.
 *   - D must be 128 and the block / page size 128; Hq / Hkv must be one of
 *     1, 2, 4, 8, 16; 1 <= topk <= 32 (the pages support D = 128 only and
 *     qhead_per_kv in {1, 2, 4, 8, 16}, topk in {4, 8, 16, 32}).
 *   - Index values outside [0, nblk) and page-table entries outside
 *     [0, num_pages) are treated as unused slots (no device-side error).
 *     The slots of one index row must name distinct blocks; repeated ids
 *     give unspecified results.
 *   - A prebuilt k2q CSR given to a forward must be what the matching
 *     msa_build_k2q_csr* call wrote for the same q2k and sizes. Any other
 *     contents give unspecified results, but every access stays inside the
 *     tensors: a row_ptr that is not non-decreasing within [0, rows * topk]
 *     (rows = B * Sq, or total_q) makes the kv-centric pass compute no partial
 *     at all, and an entry whose query lies outside its row's sequence, or
 *     whose slot lies outside [0, topk), is skipped.
 *   - Every forward entry point takes (lse_temperature_scale, lse_temperature):
 *     lse_temperature NULL skips the temperature-scaled LSE; otherwise it is an
 *     fp32 output in the layout of lse and lse_temperature_scale = T must be
 *     positive and finite. T = 1 gives exactly the bits of lse. (The page's
 *     binding returns lse itself for T = 1; the Python binding here does the
 *     same unless asked to compute it.)
 *   - Return value: MSA_OK, or an error code with a message available from
 *     msa_last_error(). Argument errors are detected on the host before any
 *     launch, and then nothing is written.
 */
#ifndef MSA_H
#define MSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum msa_status {
  MSA_OK = 0,
  MSA_ERR_INVALID_VALUE = 1, /* null / misaligned pointer, bad size, workspace too small */
  MSA_ERR_NOT_SUPPORTED = 2, /* D != 128, block != 128, Hq/Hkv or topk unsupported */
  MSA_ERR_HIP = 3            /* a HIP launch or runtime call failed */
};

enum msa_path {
  MSA_PATH_AUTO = 0,      /* kv-centric for large problems whose selected blocks each serve
                             two or more (query, slot) entries on average, else q-centric */
  MSA_PATH_QCENTRIC = 1,  /* one fused pass per (b, hkv, q) index row */
  MSA_PATH_KVCENTRIC = 2, /* CSR-driven per-block partials + LSE merge kernel */
  MSA_PATH_DECODE = 3,    /* paged only: one pass over the union of the blocks that
                             the Sq index rows of a (b, hkv) select, each block
                             read once; needs Sq <= 16 and Sq * topk <= 512 */
  MSA_PATH_TILE = 4       /* contiguous only: a workgroup per tile of consecutive
                             queries of one (b, hkv) streams the union of their
                             blocks once (for selections where many nearby queries
                             share blocks) */
};

/* K/V element type (kv_dtype of every forward entry point). */
enum msa_dtype {
  MSA_DTYPE_BF16 = 0,     /* bf16 K/V */
  MSA_DTYPE_FP8_E4M3 = 1  /* the fp8 KV cache of sparse_atten_func: OCP float8_e4m3fn bytes,
                             no scale, widened exactly to bf16 for both products, so the
                             result equals the bf16 path on the dequantized K/V bit for
                             bit; K/V tensors keep their shapes with 1-byte elements.
                             The q-centric and kv-centric kernels read it; the decode and
                             query-tile paths return MSA_ERR_NOT_SUPPORTED. For the dense
                             decode (msa_paged_decode_run) it is the pages' fp8 decode:
                             Q, K and V fp8, see there */
};

/*
 * Sparse forward, contiguous K/V (sparse_atten_func, dense KV layout).
 *   q        bf16 [B, Sq, Hq, D]
 *   k, v     bf16 [B, Skv, Hkv, D]       Skv % blk_kv == 0, nblk = Skv / blk_kv
 *   q2k      int32 [B, Hkv, Sq, topk]
 *   csr_row_ptr, csr_q_idx, csr_slot
 *            optional prebuilt k2q CSR from msa_build_k2q_csr (all three or
 *            none); used by the kv-centric path, ignored by the q-centric
 *            one. When NULL the kv-centric path builds it in the workspace.
 *   causal   0 none, 1 bottom-right (limit q + Skv - Sq)
 *   softmax_scale  <= 0 selects D^-0.5
 *   path     enum msa_path. The kv-centric path keeps one int per CSR row
 *            (B * nblk rows per KV head) in LDS, at most 16384: a longer batch
 *            runs in sub-batches of floor(16384 / nblk) whole sequences (the
 *            workspace covers one), a prebuilt CSR is then refused, and a
 *            single sequence of more than 16384 blocks returns
 *            MSA_ERR_NOT_SUPPORTED (the automatic path then takes the
 *            q-centric one).
 *   kv_dtype enum msa_dtype
 *   o        bf16 [B, Sq, Hq, D]   (out)
 *   lse      fp32 [B, Hq, Sq]      (out)
 *   lse_temperature_scale, lse_temperature   fp32 [B, Hq, Sq] or NULL (out)
 *   workspace / workspace_bytes   at least msa_sparse_fwd_workspace_size(...)
 */
size_t msa_sparse_fwd_workspace_size(int B, int Sq, int Skv, int Hq, int Hkv, int D, int topk,
                                     int blk_kv, int path);
/* The path msa_sparse_fwd takes for these sizes when given `path` (resolves
 * MSA_PATH_AUTO; other values are returned unchanged). */
int msa_sparse_fwd_path(int B, int Sq, int Skv, int Hq, int Hkv, int topk, int path);
int msa_sparse_fwd(const void* q, const void* k, const void* v, const int32_t* q2k,
                   const int32_t* csr_row_ptr, const int32_t* csr_q_idx, const int32_t* csr_slot,
                   int B, int Sq, int Skv, int Hq, int Hkv, int D, int topk, int blk_kv, int causal,
                   float softmax_scale, int path, int kv_dtype, void* o, float* lse,
                   float lse_temperature_scale, float* lse_temperature, void* workspace,
                   size_t workspace_bytes, void* stream);

/*
 * kv-block -> query CSR (build_k2q_csr on the page "MSA interface.py";
 * bit-exact checked by test_k2q_csr_builder_matches_torch_reference on the
 * test page). Row r = b * num_kv_blocks + s of KV head hkv lists the global
 * query ids b * Sq + q whose index row holds block s, ascending in q and
 * then in slot t; csr_slot holds that t.
 *   q2k       int32 [B, Hkv, Sq, topk]
 *   row_ptr   int32 [Hkv, B * num_kv_blocks + 1]   (out)
 *   q_idx     int32 [Hkv, B * Sq * topk]           (out; entries past the row
 *                                                   total are unspecified)
 *   slot      int32 [Hkv, B * Sq * topk] or NULL   (out)
 *   workspace at least msa_build_k2q_csr_workspace_size(...)
 * Deterministic: every call writes the same bits.
 */
size_t msa_build_k2q_csr_workspace_size(int B, int Hkv, int Sq, int topk, int num_kv_blocks);
int msa_build_k2q_csr(const int32_t* q2k, int B, int Hkv, int Sq, int topk, int num_kv_blocks,
                      int32_t* row_ptr, int32_t* q_idx, int32_t* slot, void* workspace,
                      size_t workspace_bytes, void* stream);

/*
 * Variable-length batches: the packed form of sparse_atten_func and
 * build_k2q_csr on the page "MSA interface.py" (cu_seqlens_q / cu_seqlens_k).
 * Sequence b owns the query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 and the
 * key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1. Its block ids count from its
 * first key (block s = its keys 128 s .. 128 s + 127; the last block may be
 * partial), valid ids are [0, ceil(Skv_b / 128)), and the causal limit is
 * q + Skv_b - Sq_b with q the row's position inside its sequence: each sequence
 * is the definition at the top of this file with B = 1. Sequences may be empty.
 *   q             bf16 [total_q, Hq, D]
 *   k, v          bf16 [total_k, Hkv, D]   (may be NULL when total_k == 0)
 *   q2k           int32 [Hkv, total_q, topk]
 *   cu_seqlens_q  int32 [B + 1] (device): 0 = cu[0] <= cu[1] <= ... <= cu[B] = total_q
 *   cu_seqlens_k  int32 [B + 1] (device): likewise, ending at total_k. Prefix sums
 *                 that break these rules give unspecified results, but every
 *                 access stays inside the tensors.
 *   csr_row_ptr, csr_q_idx, csr_slot, csr_total_rows
 *                 optional prebuilt CSR from msa_build_k2q_csr_varlen over
 *                 csr_total_rows rows (the three pointers all or none;
 *                 1 <= csr_total_rows <= floor(total_k / 128) + B); used by the
 *                 kv-centric path only
 *   path          MSA_PATH_AUTO, MSA_PATH_QCENTRIC or MSA_PATH_KVCENTRIC
 *                 (MSA_ERR_NOT_SUPPORTED for the tile and decode paths)
 *   kv_dtype      enum msa_dtype
 *   o             bf16 [total_q, Hq, D]   (out)
 *   lse           fp32 [total_q, Hq]      (out; the packed layout of the page)
 *   lse_temperature_scale, lse_temperature   fp32 [total_q, Hq] or NULL (out)
 *   workspace     at least msa_sparse_fwd_varlen_workspace_size(...)
 * total_q == 0 returns MSA_OK without touching anything.
 */
size_t msa_sparse_fwd_varlen_workspace_size(int B, int total_q, int total_k, int Hq, int Hkv,
                                            int D, int topk, int blk_kv, int path);
int msa_sparse_fwd_varlen_path(int B, int total_q, int total_k, int Hq, int Hkv, int topk,
                               int path);
int msa_sparse_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* q2k,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          const int32_t* csr_row_ptr, const int32_t* csr_q_idx,
                          const int32_t* csr_slot, int csr_total_rows, int B, int total_q,
                          int total_k, int Hq, int Hkv, int D, int topk, int blk_kv, int causal,
                          float softmax_scale, int path, int kv_dtype, void* o, float* lse,
                          float lse_temperature_scale, float* lse_temperature, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * k2q CSR of a variable-length batch (build_k2q_csr with cu_seqlens and
 * total_rows). Row rowbase[b] + s, with rowbase[b] the sum over b' < b of
 * ceil(Skv_b' / 128), lists for KV head hkv the global query ids g of sequence
 * b whose index row q2k[hkv][g][:] holds block s, ascending in g and then in
 * slot t; slot holds that t.
 *   q2k          int32 [Hkv, total_q, topk]
 *   cu_seqlens_q, cu_seqlens_k   as msa_sparse_fwd_varlen
 *   total_rows   sum over b of ceil(Skv_b / 128), computed by the caller from its
 *                lengths (entries of rows >= total_rows are dropped, rows past
 *                the true count stay empty)
 *   row_ptr      int32 [Hkv, total_rows + 1]   (out)
 *   q_idx, slot  int32 [Hkv, total_q * topk]   (out; slot may be NULL)
 *   workspace    at least msa_build_k2q_csr_varlen_workspace_size(...)
 * Deterministic: every call writes the same bits.
 */
size_t msa_build_k2q_csr_varlen_workspace_size(int B, int Hkv, int total_q, int topk,
                                               int total_rows);
int msa_build_k2q_csr_varlen(const int32_t* q2k, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, int B, int Hkv, int total_q, int total_k,
                             int topk, int total_rows, int32_t* row_ptr, int32_t* q_idx,
                             int32_t* slot, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sparse forward, paged K/V (sparse_atten_func with page_table / seqused_k,
 * and the split-KV decode of sparse_decode_atten_func on the page
 * "MSA interface.py"; paging as in pack_paged_kv on the test page).
 *   q           bf16 [B, Sq, Hq, D]
 *   k_pool, v_pool  bf16 [num_pages, Hkv, page_size, D]
 *   page_table  int32 [B, max_pages]: logical block s of sequence b is page
 *               page_table[b][s]
 *   seqused_k   int32 [B]: valid KV length of each sequence
 *               (1 <= seqused_k[b] <= max_pages * page_size; keys at or past it
 *               are masked and never influence the result)
 *   q2k         int32 [B, Hkv, Sq, topk], valid ids [0, max_pages)
 *   causal      bottom-right with the limit q + seqused_k[b] - Sq
 *   num_splits  0 = automatic; else the number of KV splits, each a partial pass
 *               merged afterwards by log-sum-exp. q-centric: each index row's
 *               slots are split (clamped to 1..topk); decode: the union of the
 *               blocks of a (b, hkv) is split (clamped to 1..min(Sq*topk, 64));
 *               kv-centric: ignored (its partials are per block already)
 *   path        MSA_PATH_AUTO, MSA_PATH_QCENTRIC, MSA_PATH_KVCENTRIC or
 *               MSA_PATH_DECODE. Auto takes the kv-centric path under the rule of
 *               msa_sparse_fwd with max_pages blocks per sequence (large problems
 *               whose blocks each serve two or more (query, slot) entries, e.g. a
 *               long prefill), else the q-centric one (decode batches).
 *               kv-centric: the sparse_atten_func pipeline (k2q CSR, per-block
 *               partials, combine) with each block read through the page table;
 *               B * max_pages CSR rows, in sub-batches of floor(16384 / max_pages)
 *               sequences past 16384, MSA_ERR_NOT_SUPPORTED when max_pages > 16384.
 *               Decode reads each distinct block of a (b, hkv) once: for index
 *               rows that share blocks; MSA_ERR_NOT_SUPPORTED when Sq > 16 or
 *               Sq * topk > 512.
 *   kv_dtype    enum msa_dtype (fp8 with the q-centric and kv-centric paths)
 *   o, lse, lse_temperature_scale, lse_temperature   as msa_sparse_fwd
 *   workspace   at least msa_paged_sparse_fwd_workspace_size(...) with the same
 *               num_splits and path (zero when one q-centric or decode split
 *               results; the kv-centric path always takes one)
 * A block past seqused_k[b], or whose page id is outside [0, num_pages), adds
 * nothing to a row on every path; nothing of it is read.
 * Duplicate ids within one index row: the decode path counts each block once;
 * the q-centric and kv-centric paths require distinct ids.
 */
size_t msa_paged_sparse_fwd_workspace_size(int B, int Sq, int Hq, int Hkv, int D, int topk,
                                           int page_size, int max_pages, int num_splits,
                                           int path);
/* The kernel msa_paged_sparse_fwd runs for these sizes (resolves MSA_PATH_AUTO)
 * and the number of splits it uses (0 for invalid sizes). */
int msa_paged_sparse_fwd_path(int B, int Sq, int Hkv, int topk, int max_pages, int path);
int msa_paged_sparse_fwd_splits(int B, int Sq, int Hkv, int topk, int max_pages, int num_splits,
                                int path);
int msa_paged_sparse_fwd(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, const int32_t* seqused_k, const int32_t* q2k,
                         int B, int Sq, int Hq, int Hkv, int D, int topk, int page_size,
                         int num_pages, int max_pages, int causal, float softmax_scale,
                         int num_splits, int path, int kv_dtype, void* o, float* lse,
                         float lse_temperature_scale, float* lse_temperature, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Sparse forward, paged K/V with a packed variable-length query batch: the paged
 * form of sparse_atten_func (page_table and seqused_k with cu_seqlens_q) on the
 * page "MSA interface.py"; the test page's test_sparse_page_atten runs it.
 *   q             bf16 [total_q, Hq, D]; sequence b's queries are rows
 *                 cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 *   k_pool, v_pool, page_table, seqused_k, num_pages, max_pages
 *                 as msa_paged_sparse_fwd (seqused_k[b] keys for sequence b)
 *   cu_seqlens_q  int32 [B+1] on the device, non-decreasing from 0 to total_q
 *   q2k           int32 [Hkv, total_q, topk], valid ids [0, max_pages)
 *   causal        bottom-right with the limit q + seqused_k[b] - Sq_b, q counted
 *                 from the sequence's first query
 *   num_splits    q-centric: 0 = automatic (as msa_paged_sparse_fwd with total_q
 *                 query rows), else the number of slot splits (clamped to 1..topk),
 *                 merged by log-sum-exp; kv-centric: ignored
 *   path          MSA_PATH_AUTO, MSA_PATH_QCENTRIC or
 *                 MSA_PATH_KVCENTRIC (max_pages CSR rows per sequence, B * max_pages
 *                 at most 16384, else MSA_ERR_NOT_SUPPORTED); auto takes the
 *                 kv-centric path under the rule of msa_sparse_fwd with total_q
 *                 queries over B * max_pages rows
 *   kv_dtype      enum msa_dtype
 *   o             bf16 [total_q, Hq, D]   (out)
 *   lse           fp32 [total_q, Hq]      (out)
 *   lse_temperature_scale, lse_temperature   fp32 [total_q, Hq] or NULL (out)
 *   workspace     at least msa_paged_sparse_fwd_varlen_workspace_size(...) with the
 *                 same num_splits and path (zero for one q-centric split)
 * A block past seqused_k[b], or whose page id is outside [0, num_pages), adds nothing.
 * Index rows must hold distinct ids. total_q = 0 writes nothing and returns MSA_OK.
 */
size_t msa_paged_sparse_fwd_varlen_workspace_size(int B, int total_q, int Hq, int Hkv, int D,
                                                  int topk, int page_size, int max_pages,
                                                  int num_splits, int path);
/* The path msa_paged_sparse_fwd_varlen takes for these sizes (resolves MSA_PATH_AUTO)
 * and the number of splits it uses (1 on the kv-centric path, 0 for invalid sizes). */
int msa_paged_sparse_fwd_varlen_path(int B, int total_q, int Hkv, int topk, int max_pages,
                                     int path);
int msa_paged_sparse_fwd_varlen_splits(int B, int total_q, int Hkv, int topk, int max_pages,
                                       int num_splits, int path);
int msa_paged_sparse_fwd_varlen(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* page_table, const int32_t* seqused_k,
                                const int32_t* cu_seqlens_q, const int32_t* q2k, int B,
                                int total_q, int Hq, int Hkv, int D, int topk, int page_size,
                                int num_pages, int max_pages, int causal, float softmax_scale,
                                int num_splits, int path, int kv_dtype, void* o, float* lse,
                                float lse_temperature_scale, float* lse_temperature,
                                void* workspace, size_t workspace_bytes, void* stream);

/*
 * msa_paged_sparse_fwd without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops and
 * harnesses that forbid hipMalloc. Arguments, results and errors are those of
 * msa_paged_sparse_fwd, and so are the kernels (results bit for bit equal), except
 * that MSA_PATH_AUTO never resolves to the kv-centric path here (it takes the
 * q-centric one instead): that path's partials outgrow the scratch on the problems
 * it is chosen for.
 *   Scratch: the split partials use a device array inside the library of
 *   MSA_NOALLOC_SCRATCH_BYTES per GPU, which each GPU the library runs on holds
 *   until the process ends. Its device address is looked up on the first call
 *   on a device (hipGetSymbolAddress, a set-up step that may load the code
 *   object there); later calls allocate nothing and call no allocating routine.
 *   Limit: calls whose split partials need more than MSA_NOALLOC_SCRATCH_BYTES
 *   (msa_paged_sparse_fwd_workspace_size with the same sizes, num_splits and
 *   path) return MSA_ERR_INVALID_VALUE before any launch. One split (the
 *   automatic choice on decode batches of 1024 or more (b, hkv, q) rows) needs
 *   no scratch at all.
 *   Concurrency: every call on one GPU shares that GPU's array, and each call
 *   overwrites what the previous one left there; calls that overlap in time on
 *   one GPU (different streams, or several threads) race and give undefined
 *   results. Serialise them on one stream.
 */
#define MSA_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int msa_paged_sparse_fwd_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* page_table, const int32_t* seqused_k,
                                 const int32_t* q2k, int B, int Sq, int Hq, int Hkv, int D,
                                 int topk, int page_size, int num_pages, int max_pages, int causal,
                                 float softmax_scale, int num_splits, int path, int kv_dtype,
                                 void* o, float* lse, float lse_temperature_scale,
                                 float* lse_temperature, void* stream);

/*
 * Dense paged decode with a plan/run split-KV schedule: the q2k = None path of
 * sparse_decode_atten_func and SparseDecodePagedAttentionWrapper.plan / .run on
 * the page "MSA interface.py". Every query row attends to all keys of its
 * sequence (j < seqused_k[b], causal limit q + seqused_k[b] - Sq): the definition
 * at the top of this file with every block selected. Q bf16 [B, Sq, Hq, D]
 * (Sq <= 16; fp8 below), K/V bf16 pools [num_pages, Hkv, 128, D], O [B, Sq, Hq, D],
 * LSE [B, Hq, Sq]. A workgroup takes one (sequence, chunk of pages, KV head) and
 * reads each page once for all Sq query rows; a sequence cut into several chunks
 * gets fp32 partial rows, merged by log-sum-exp afterwards.
 *
 * msa_paged_decode_plan_init (host only) fixes the chunk size and the layout of a
 * plan buffer (device memory the caller allocates, `bytes` long, 256-byte
 * aligned): the schedule arrays and the partial-row workspace.
 *   max_seqlen_k       upper bound of seqused_k (sizes the plan)
 *   max_grid_size      0 = two workgroups per compute unit: the target number of
 *                      (sequence, chunk, KV head) items when splitting
 *   fixed_split_pages  0 = automatic; else the chunk size in pages (1..512)
 *   disable_split_kv   one chunk per sequence (needs max_seqlen_k <= 512 pages)
 * msa_paged_decode_plan builds the schedule on the device from seqused_k on
 * `stream`, into the plan buffer; it stays valid while seqused_k does not change,
 * and any number of runs may use it. msa_paged_decode_run runs the decode. A run
 * with a seqused_k changed since the plan stays inside the tensors (page counts
 * are clamped to max_pages when planned, key counts when run) but its results
 * are unspecified; a run on a buffer that msa_paged_decode_plan has not filled
 * for this plan reads garbage indices and is undefined behaviour.
 * The schedule arrays (int32, at the byte offsets in the plan): kv_pages[B]
 * (ceil(seqused / 128)), split_counts[B] (chunks of each sequence), o_indptr[B+1]
 * (first partial row of each sequence; it advances by Sq * chunks),
 * merge_indptr[B*Sq+1] (the partial rows of query row (b, q) are
 * merge_indptr[b*Sq+q] + 0 .. split_counts[b]-1), work_items (int4: sequence,
 * chunk, first page, pages) and work_count[1].
 */
typedef struct msa_decode_plan {
  int batch, seqlen_q, num_qo_heads, num_kv_heads, max_pages;
  int kv_chunk_size_pages; /* pages per chunk */
  int split_kv;            /* 0: every sequence in one chunk */
  int padded_work_count;   /* batch * ceil(max_pages / chunk): bound on the work items */
  int64_t partial_rows;    /* capacity of the partial rows: batch * Sq * max chunks */
  size_t kv_pages, split_counts, o_indptr, merge_indptr, work_offsets, work_items,
      work_count, o_partial, lse_partial, lse_t_partial; /* byte offsets in the buffer */
  size_t bytes;            /* plan buffer size */
} msa_decode_plan;

int msa_paged_decode_plan_init(int B, int Sq, int Hq, int Hkv, int D, int page_size,
                               int max_seqlen_k, int max_grid_size, int fixed_split_pages,
                               int disable_split_kv, msa_decode_plan* plan);
int msa_paged_decode_plan(const int32_t* seqused_k, const msa_decode_plan* plan, void* buffer,
                          size_t buffer_bytes, void* stream);
/* num_pages: pool size (page ids outside [0, num_pages) read as unused blocks);
 * the page table is [B, plan->max_pages].
 * dtype: MSA_DTYPE_BF16 (Q, K, V bf16) or MSA_DTYPE_FP8_E4M3, the fp8 decode of
 *   sparse_decode_atten_func as the test page "test_sparse_atten.py" checks it
 *   (`_decode_paged_dense_reference`): Q [B, Sq, Hq, D] and the K/V pools are OCP
 *   float8_e4m3fn bytes (no scale), the unnormalised probabilities are rounded to
 *   e4m3 (nearest, ties to even) before the P V product while the row sum and the
 *   LSE use the unrounded ones; O stays bf16. Only for Sq * Hq / Hkv <= 128
 *   (else MSA_ERR_NOT_SUPPORTED). The rounding point is the kernel's running
 *   reference maximum rather than the row's final maximum, which changes results
 *   within the e4m3 rounding (the page allows 0.125 on O and 2e-3 on the LSE).
 * Other arguments as msa_paged_sparse_fwd. */
int msa_paged_decode_run(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, const int32_t* seqused_k,
                         const msa_decode_plan* plan, void* buffer, size_t buffer_bytes,
                         int num_pages, int dtype, int causal, float softmax_scale, void* o,
                         float* lse, float lse_temperature_scale, float* lse_temperature,
                         void* stream);

/*
 * Profiling hook (for benchmarks): when both are non-NULL, every later
 * forward call on this thread records `before` and `after` (hipEvent_t handles
 * created by the caller) on its stream immediately around the launch of its
 * dominant kernel -- the kv-centric per-block kernel, the q-centric kernel or
 * the paged (q-centric or decode) kernel -- so the caller can read that kernel's duration with
 * hipEventElapsedTime. NULL, NULL switches it off. Returns MSA_OK, or
 * MSA_ERR_INVALID_VALUE if exactly one is NULL.
 */
int msa_set_profiling_events(void* before, void* after);

/* Message of the last failed call on this thread ("" if none). */
const char* msa_last_error(void);

/* Library version string. */
const char* msa_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MSA_H */
