// C ABI of libmsa: host-side validation, workspace layout and dispatch.
// Declarations and the contract of every entry point are in include/msa.h.
#include "../../include/msa.h"
#include "msa_internal.hpp"

#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>

using namespace msa;

namespace {

thread_local std::string g_last_error;
thread_local hipEvent_t g_prof_before = nullptr;
thread_local hipEvent_t g_prof_after = nullptr;

// records the caller's profiling event (if set) on the launch stream
void prof_mark(hipEvent_t ev, hipStream_t st) {
  if (ev) (void)hipEventRecord(ev, st);
}

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* where) {
  return fail(MSA_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

bool qpk_supported(int qpk) { return qpk == 1 || qpk == 2 || qpk == 4 || qpk == 8 || qpk == 16; }

// Checks shared by the forward entry points; returns MSA_OK or an error code.
int check_common(int B, int Sq, int Hq, int Hkv, int D, int topk, int blk) {
  if (B <= 0 || Sq <= 0 || Hq <= 0 || Hkv <= 0 || topk <= 0)
    return fail(MSA_ERR_INVALID_VALUE, "B, Sq, Hq, Hkv and topk must be positive");
  if (D != kD) return fail(MSA_ERR_NOT_SUPPORTED, "head dim %d not supported (only 128)", D);
  if (blk != kBlk) return fail(MSA_ERR_NOT_SUPPORTED, "block/page size %d not supported (only 128)", blk);
  if (Hq % Hkv != 0) return fail(MSA_ERR_INVALID_VALUE, "Hq (%d) must be a multiple of Hkv (%d)", Hq, Hkv);
  if (!qpk_supported(Hq / Hkv))
    return fail(MSA_ERR_NOT_SUPPORTED, "qhead_per_kv %d not supported (1, 2, 4, 8 or 16)", Hq / Hkv);
  if (topk > kMaxTopk) return fail(MSA_ERR_NOT_SUPPORTED, "topk %d not supported (1..32)", topk);
  if (static_cast<long long>(B) * Sq * topk > 0x7FFFFFFFLL)
    return fail(MSA_ERR_INVALID_VALUE, "B*Sq*topk exceeds the int32 index range");
  return MSA_OK;
}

// Automatic choice. The q-centric kernel works through (query, KV head, block) units,
// each a 64 KiB K/V block read through the caches and multiplied for the qhead_per_kv
// heads (padded to 16 matrix columns), so its time grows with the unit count whatever
// qhead_per_kv is. The kv-centric path reads each selected block once per chunk of
// ~2048 (query, head) rows and pays a bf16 partial round trip per (query, head, slot),
// after a fixed chain of ~45 us of CSR, item and combine launches. Measured on one
// MI355X (B 1, Hkv 4, Sq = Skv 256-8192, qhead_per_kv 1/4/16, topk 8/16, causal or
// not), the kv-centric path is the faster one from 32768 units on, by up to 12x at
// qhead_per_kv 1, and at most 17% slower just past that point at qhead_per_kv 16.
// That needs each selected block to serve several queries: a kv-centric item reads its
// block once for the queries that selected it. Batches of short query sets over long
// keys select each block about once (entries per CSR row = Sq * topk / blocks), and
// there the q-centric kernel was faster (Hkv 4, 64 query heads, topk 16, causal): 0.38
// against 0.64 ms at 0.25 entries per row (64 sequences of 8 queries over 65 536
// keys), 1.27 against 1.55 ms at 1 (64 of 32 over 65 536); from 2 entries per row on
// the kv-centric path was as fast or faster (0.34 against 0.32 ms for 64 of 8 over
// 8192, 1.15 against 0.80 ms for 16 of 128 over 65 536, at 4).
// A sequence with more blocks than the LDS-resident CSR passes hold takes the q-centric
// path; a batch with more rows in all runs the kv-centric path in sub-batches.
constexpr long long kKvMinUnits = 32768;
constexpr long long kKvMinEntriesPerRow = 2;
long long qcentric_units(long long nq, int Hkv, int topk, long long nblk) {
  return nq * Hkv * std::min<long long>(topk, nblk);  // blocks past the last one are unused
}
// nq query rows selecting among nrows CSR rows of nblk blocks per sequence (per KV head)
bool kv_pays(long long nq, int Hkv, int topk, long long nblk, long long nrows) {
  return qcentric_units(nq, Hkv, topk, nblk) >= kKvMinUnits &&
         nq * std::min<long long>(topk, nblk) >= kKvMinEntriesPerRow * nrows;
}
int resolve_path(int path, int B, int Sq, int Skv, int Hq, int Hkv, int topk) {
  if (path == MSA_PATH_QCENTRIC || path == MSA_PATH_KVCENTRIC || path == MSA_PATH_TILE) return path;
  (void)Hq;
  const long long nblk = Skv / kBlk;
  if (nblk > kMaxCsrRows ||
      !kv_pays(static_cast<long long>(B) * Sq, Hkv, topk, nblk, static_cast<long long>(B) * nblk))
    return MSA_PATH_QCENTRIC;
  return MSA_PATH_KVCENTRIC;
}

// The kv-centric passes hold one int per CSR row in LDS, so a batch of more than
// kMaxCsrRows rows (B * Skv / 128) runs as consecutive sub-batches of this many whole
// sequences (a sequence's queries select only its own blocks); 0 when one sequence alone
// has too many blocks.
int kv_sub_batch(int B, int nblk) {
  return nblk > kMaxCsrRows ? 0 : std::min(B, kMaxCsrRows / nblk);
}

// Varlen batches: the same rule with the packed sizes. The lengths are on the device,
// so the host bounds a sequence's blocks by ceil(total_k / 128) and the CSR row count
// by floor(total_k / 128) + B (each sequence adds at most one partial block).
long long varlen_rows_bound(int B, long long total_k) { return total_k / kBlk + B; }
int resolve_varlen_path(int path, int B, long long total_q, long long total_k, int Hkv,
                        int topk) {
  if (path != MSA_PATH_AUTO) return path;
  if (total_k == 0 || varlen_rows_bound(B, total_k) > kMaxCsrRows ||
      !kv_pays(total_q, Hkv, topk, (total_k + kBlk - 1) / kBlk, varlen_rows_bound(B, total_k)))
    return MSA_PATH_QCENTRIC;
  return MSA_PATH_KVCENTRIC;
}

// K/V element type: bf16 or the fp8 e4m3fn cache; the direct-to-LDS kernels (paged
// decode, query tile) read bf16 only.
int check_kv_dtype(int kv_dtype, int path_taken) {
  if (kv_dtype != MSA_DTYPE_BF16 && kv_dtype != MSA_DTYPE_FP8_E4M3)
    return fail(MSA_ERR_INVALID_VALUE, "unknown kv_dtype %d", kv_dtype);
  if (kv_dtype == MSA_DTYPE_FP8_E4M3 && (path_taken == MSA_PATH_DECODE || path_taken == MSA_PATH_TILE))
    return fail(MSA_ERR_NOT_SUPPORTED, "the %s path reads bf16 K/V only",
                path_taken == MSA_PATH_DECODE ? "decode" : "query-tile");
  return MSA_OK;
}

// Temperature-scaled LSE request: no buffer = off; else T must be positive and finite.
int check_temperature(float scale, const float* lse_t) {
  if (!lse_t) return MSA_OK;
  if (!(scale > 0.f) || !isfinite(scale))
    return fail(MSA_ERR_INVALID_VALUE, "lse_temperature_scale must be positive and finite");
  if (!aligned(lse_t, 4)) return fail(MSA_ERR_INVALID_VALUE, "misaligned lse_temperature pointer");
  return MSA_OK;
}

// Streams of the kv-centric item order: one per KV head, up to one per XCD. With a
// single KV head one stream keeps every running item in one query range, so that the
// Q rows they gather share the last-level cache (measured faster than 8 query-range
// streams at 393 216 queries x 2 heads: 2.14 against 2.23 ms per step).
int kv_streams(int Hkv) { return Hkv >= 8 ? 8 : (Hkv >= 4 ? 4 : (Hkv >= 2 ? 2 : 1)); }

// Entries per kv-centric work item: kKvChunkRows (query, head) rows.
int chunk_entries_for(int qpk) { return std::min(kKvMaxEntries, kKvChunkRows / qpk); }

struct KvLayout {
  size_t row_ptr, q_idx, csr_ws, items, items_by_q, sort_counts, o_part, lse_part, lse_t_part,
      total;
  long long max_items;
};

// nq query rows (B * Sq, or total_q), nrows CSR rows
KvLayout kv_layout(long long nq, long long nrows, int Hq, int Hkv, int topk) {
  const long long cap = nq * topk;
  KvLayout L;
  size_t off = 0;
  L.row_ptr = off; off += align256(Hkv * (nrows + 1) * 4);
  L.q_idx = off; off += align256(Hkv * cap * 4);
  L.csr_ws = off;
  off += align256(csr_workspace_bytes(1, Hkv, static_cast<int>(nq), topk, static_cast<int>(nrows)));
  // one slot per possible item (kv_item_slot): per KV head cap / chunk + nrows + 1
  L.max_items = static_cast<long long>(Hkv) * (cap / chunk_entries_for(Hq / Hkv) + nrows + 1);
  L.items = off; off += align256(L.max_items * 16);
  L.items_by_q = off; off += align256(L.max_items * 16);
  L.sort_counts = off; off += align256(kKvSortInts * 4);
  L.o_part = off; off += align256(static_cast<size_t>(cap) * Hq * kD * 2);
  L.lse_part = off; off += align256(static_cast<size_t>(cap) * Hq * 8);
  L.lse_t_part = off; off += align256(static_cast<size_t>(cap) * Hq * 4);
  L.total = off;
  return L;
}

// Paged plan: which kernel and how many KV splits. MSA_PATH_AUTO takes the
// kv-centric path under the contiguous rule (max_pages blocks per sequence), else the
// q-centric kernel: on the 32 x 8-query decode workload with random per-query
// blocks it measured faster than the union (decode) kernel, which reads each
// distinct block of a (b, hkv) once and pays off when the Sq index rows share
// blocks; the caller asks for it explicitly. The kv-centric path does not split
// (its partials are per block already). The decode kernel splits the union
// into `splits` contiguous shares; the q-centric kernel splits each index row's
// slots. Automatic splits aim at about three workgroups per compute unit
// (decode) or about 1024 single-wave workgroups (q-centric: on the 32 x 8 x 4
// decode workload one split, 1024 waves, measured fastest; 2, 4 and 8 splits
// were 5-15% slower and add the combine pass).
struct PagedPlan {
  int path;
  int splits;
};

// q-centric split count for `rows` (query, KV head) rows: num_splits (0 = about 1024
// single-wave workgroups, at most 8), clamped to 1..topk
int qcentric_splits(long long rows, int topk, int num_splits) {
  long long s = num_splits;
  if (s <= 0) s = std::min<long long>((1024 + rows - 1) / rows, 8);
  return static_cast<int>(std::max<long long>(1, std::min<long long>(s, topk)));
}

PagedPlan paged_plan(int B, int Sq, int Hkv, int topk, int max_pages, int num_splits, int path) {
  PagedPlan pl;
  if (path == MSA_PATH_AUTO)
    path = max_pages <= kMaxCsrRows &&
                   kv_pays(static_cast<long long>(B) * Sq, Hkv, topk, max_pages,
                           static_cast<long long>(B) * max_pages)
               ? MSA_PATH_KVCENTRIC
               : MSA_PATH_QCENTRIC;
  pl.path = path;
  if (path == MSA_PATH_KVCENTRIC) {
    pl.splits = 1;
  } else if (path == MSA_PATH_DECODE) {
    const long long cap = std::min<long long>(static_cast<long long>(Sq) * topk, kMaxDecodeSplits);
    long long s = num_splits;
    if (s <= 0) {
      const long long pairs = static_cast<long long>(B) * Hkv;
      s = (3LL * device_cu_count() + pairs - 1) / pairs;
    }
    pl.splits = static_cast<int>(std::max<long long>(1, std::min(s, cap)));
  } else {
    pl.splits = qcentric_splits(static_cast<long long>(B) * Hkv * Sq, topk, num_splits);
  }
  return pl;
}

// q-centric and decode: fp32 partials [splits][rows][D], then the split LSEs and
// temperature-scaled LSEs [splits][rows], rows = B * Sq * Hq. kv-centric: the
// contiguous path's workspace for its largest sub-batch.
size_t paged_workspace(int B, int Sq, int Hq, int Hkv, int topk, int max_pages,
                       const PagedPlan& pl) {
  if (pl.path == MSA_PATH_KVCENTRIC) {
    const int bc = kv_sub_batch(B, max_pages);
    if (bc == 0) return 0;
    return kv_layout(static_cast<long long>(bc) * Sq, static_cast<long long>(bc) * max_pages, Hq,
                     Hkv, topk).total;
  }
  const int splits = pl.splits;
  if (splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(B) * Sq * Hq;
  return align256(splits * rows * kD * 4) + 2 * align256(splits * rows * 4);
}

// The kv-centric pipeline: k2q CSR (unless given) and the work items, items in key
// order, per-block partials, slot combine. `p` carries the problem (and, for a varlen
// batch, cu_q / cu_k / total sizes); vt != nullptr selects the varlen layout,
// its tables already built on the stream.
int run_kvcentric(KvParams p, const int32_t* q2k, const int32_t* csr_row_ptr,
                  const int32_t* csr_q_idx, const int32_t* csr_slot, const KvLayout& L, char* ws,
                  const VarlenTables* vt, uint16_t* o, float* lse, float* lse_t,
                  hipStream_t st) {
  const int nrows = p.nrows;
  const long long nq = vt ? p.total_q : static_cast<long long>(p.B) * p.Sq;
  const int32_t* row_ptr = csr_row_ptr;
  const int32_t* q_idx = csr_q_idx;
  const int32_t* slot = csr_slot;
  hipError_t e;
  if (L.max_items > 0x7FFFFFFFLL) return fail(MSA_ERR_INVALID_VALUE, "problem too large");
  const int chunk = chunk_entries_for(p.qpk);  // a power of two
  int chunk_shift = 0;
  while ((1 << chunk_shift) < chunk) ++chunk_shift;
  const KvSortBuffers sb = kv_sort_buffers(reinterpret_cast<int32_t*>(ws + L.sort_counts));
  int4* items = reinterpret_cast<int4*>(ws + L.items);
  // q_idx entries hold query * qdiv + slot: the library's own CSR stores each entry as
  // its index-table position (one int32, half the scatter's stores); a caller's CSR
  // holds the query ids with the slots beside them
  int qdiv = 1;
  if (!row_ptr) {
    // the order-free CSR lists the work items (one per chunk of each row) while it
    // scatters; its count pass clears the item counters
    int32_t* rp = reinterpret_cast<int32_t*>(ws + L.row_ptr);
    int32_t* qi = reinterpret_cast<int32_t*>(ws + L.q_idx);
    const KvItemEmit emit{items, L.max_items / p.Hkv, L.max_items, sb, chunk_shift};
    if (vt)
      e = launch_build_csr_varlen(q2k, *vt, p.Hkv, static_cast<int>(nq), p.topk, nrows, rp, qi,
                                  nullptr, ws + L.csr_ws, st, /*ordered=*/false, /*flat=*/true,
                                  &emit);
    else
      e = launch_build_csr(q2k, p.B, p.Hkv, p.Sq, p.topk, p.nblk, rp, qi, nullptr, ws + L.csr_ws,
                           st, /*ordered=*/false, /*flat=*/true, &emit);
    if (e != hipSuccess) return hip_fail(e, "k2q CSR build");
    row_ptr = rp; q_idx = qi; slot = nullptr;
    qdiv = p.topk;
  } else {
    e = launch_zero_ints(sb.counts, kKvSortZeroInts, reinterpret_cast<int32_t*>(items),
                         4 * L.max_items, st);
    if (e == hipSuccess)
      e = launch_kv_items(row_ptr, p.Hkv, nrows, chunk_shift, L.max_items / p.Hkv, items, q_idx,
                          nq * p.topk, nq, qdiv, sb, st);
    if (e != hipSuccess) return hip_fail(e, "kv-centric item table");
  }
  p.row_ptr = row_ptr; p.q_idx = q_idx; p.slot = slot;
  p.chunk_entries = chunk;
  p.o_part = reinterpret_cast<uint16_t*>(ws + L.o_part);
  p.lse_part = reinterpret_cast<float2*>(ws + L.lse_part);
  p.lse_t_part = lse_t ? reinterpret_cast<float*>(ws + L.lse_t_part) : nullptr;
  if (vt) {
    p.rowbase = vt->rowbase;
    p.row_seq = vt->row_seq;
  }
  // The items ordered by (KV head, first query) and cut into one stream per XCD: the
  // items running together on an XCD then gather Q rows from one narrow query range of
  // one KV head, which stays in that XCD's L2. The order-free CSR lists each row's
  // entries in ascending query tiles, so an item's first query marks where its query
  // range starts.
  int4* sorted = reinterpret_cast<int4*>(ws + L.items_by_q);
  e = launch_kv_items_by_key(items, p.Hkv, q_idx, nq * p.topk, nq, qdiv, L.max_items, sb, sorted,
                             st);
  if (e != hipSuccess) return hip_fail(e, "kv-centric item order");
  p.items = sorted;
  p.key_start = sb.key_start;
  p.stream_next = sb.next;
  p.streams = kv_streams(p.Hkv);
  prof_mark(g_prof_before, st);
  e = launch_kvcentric(p, L.max_items, st);
  prof_mark(g_prof_after, st);
  if (e != hipSuccess) return hip_fail(e, "kv-centric forward");
  if (vt) {
    const CombineVarlen cv{vt->q_rows};
    e = launch_combine_slots(p.o_part, p.lse_part, q2k, 1, static_cast<int>(nq), p.Hq, p.Hkv,
                             p.topk, 0, o, lse, st, &cv, p.lse_t_part, lse_t);
  } else {
    e = launch_combine_slots(p.o_part, p.lse_part, q2k, p.B, p.Sq, p.Hq, p.Hkv, p.topk, p.nblk, o,
                             lse, st, nullptr, p.lse_t_part, lse_t);
  }
  return e == hipSuccess ? MSA_OK : hip_fail(e, "combine");
}

}  // namespace

int msa::device_cu_count() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

extern "C" {

const char* msa_last_error(void) { return g_last_error.c_str(); }

int msa_set_profiling_events(void* before, void* after) {
  if ((before == nullptr) != (after == nullptr))
    return fail(MSA_ERR_INVALID_VALUE, "profiling events must both be set or both be NULL");
  g_prof_before = static_cast<hipEvent_t>(before);
  g_prof_after = static_cast<hipEvent_t>(after);
  return MSA_OK;
}

const char* msa_version(void) { return "msa-gfx950 0.1.0"; }

int msa_sparse_fwd_path(int B, int Sq, int Skv, int Hq, int Hkv, int topk, int path) {
  return resolve_path(path, B, Sq, Skv, Hq, Hkv, topk);
}

size_t msa_sparse_fwd_workspace_size(int B, int Sq, int Skv, int Hq, int Hkv, int D, int topk,
                                     int blk_kv, int path) {
  if (B <= 0 || Sq <= 0 || Skv <= 0 || Hq <= 0 || Hkv <= 0 || topk <= 0 || D != kD ||
      blk_kv != kBlk || Skv % kBlk || Hq % Hkv)
    return 0;
  const int which = resolve_path(path, B, Sq, Skv, Hq, Hkv, topk);
  if (which == MSA_PATH_QCENTRIC || which == MSA_PATH_TILE) return 0;
  const int bc = kv_sub_batch(B, Skv / kBlk);  // the largest sub-batch
  if (bc == 0) return 0;
  return kv_layout(static_cast<long long>(bc) * Sq, static_cast<long long>(bc) * (Skv / kBlk), Hq,
                   Hkv, topk).total;
}

int msa_sparse_fwd(const void* q, const void* k, const void* v, const int32_t* q2k,
                   const int32_t* csr_row_ptr, const int32_t* csr_q_idx, const int32_t* csr_slot,
                   int B, int Sq, int Skv, int Hq, int Hkv, int D, int topk, int blk_kv, int causal,
                   float softmax_scale, int path, int kv_dtype, void* o, float* lse,
                   float lse_temperature_scale, float* lse_temperature, void* workspace,
                   size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_common(B, Sq, Hq, Hkv, D, topk, blk_kv);
  if (rc) return rc;
  rc = check_temperature(lse_temperature_scale, lse_temperature);
  if (rc) return rc;
  const float inv_temp = lse_temperature ? 1.f / lse_temperature_scale : 1.f;
  if (Skv <= 0 || Skv % kBlk)
    return fail(MSA_ERR_INVALID_VALUE, "Skv (%d) must be a positive multiple of 128", Skv);
  if (!q || !k || !v || !q2k || !o || !lse)
    return fail(MSA_ERR_INVALID_VALUE, "null tensor pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(q2k, 4) || !aligned(lse, 4))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned tensor pointer (bf16 tensors need 16 bytes)");
  if (path != MSA_PATH_AUTO && path != MSA_PATH_QCENTRIC && path != MSA_PATH_KVCENTRIC &&
      path != MSA_PATH_TILE)
    return fail(MSA_ERR_INVALID_VALUE, "unknown path %d", path);
  const bool have_csr = csr_row_ptr || csr_q_idx || csr_slot;
  if (have_csr && !(csr_row_ptr && csr_q_idx && csr_slot))
    return fail(MSA_ERR_INVALID_VALUE, "csr_row_ptr, csr_q_idx and csr_slot go together");
  const int qpk = Hq / Hkv;
  const int nblk = Skv / kBlk;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(D));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int which = resolve_path(path, B, Sq, Skv, Hq, Hkv, topk);
  rc = check_kv_dtype(kv_dtype, which);
  if (rc) return rc;
  const int kv_fp8 = kv_dtype == MSA_DTYPE_FP8_E4M3;

  if (which == MSA_PATH_TILE) {
    if (!tile_supported(qpk, topk))
      return fail(MSA_ERR_NOT_SUPPORTED,
                  "query-tile path needs qhead_per_kv 8 or 16 and (256 / qhead_per_kv) * topk "
                  "<= %d (got qhead_per_kv %d, topk %d)", kTileMaxEntries, qpk, topk);
    TileParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = static_cast<const uint16_t*>(k);
    p.v = static_cast<const uint16_t*>(v);
    p.q2k = q2k;
    p.B = B; p.Sq = Sq; p.Skv = Skv; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk; p.topk = topk;
    p.nblk = nblk; p.causal = causal ? 1 : 0;
    p.scale_log2 = scale * kLog2e;
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.inv_temp = inv_temp;
    p.lse_t = lse_temperature;
    prof_mark(g_prof_before, st);
    hipError_t e = launch_tile(p, st);
    prof_mark(g_prof_after, st);
    return e == hipSuccess ? MSA_OK : hip_fail(e, "query-tile forward");
  }

  if (which == MSA_PATH_QCENTRIC) {
    QcParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = k;
    p.v = v;
    p.kv_fp8 = kv_fp8;
    p.q2k = q2k;
    p.B = B; p.Sq = Sq; p.Skv = Skv; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk; p.topk = topk;
    p.nblk = nblk; p.causal = causal ? 1 : 0;
    p.kv_stream = static_cast<long long>(Sq) * std::min(topk, nblk) < kKvMinEntriesPerRow * nblk;
    p.scale_log2 = scale * kLog2e;
    p.splits = 1;
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.inv_temp = inv_temp;
    p.lse_t = lse_temperature;
    prof_mark(g_prof_before, st);
    hipError_t e = launch_qcentric(p, false, st);
    prof_mark(g_prof_after, st);
    return e == hipSuccess ? MSA_OK : hip_fail(e, "q-centric forward");
  }

  // kv-centric, in sub-batches of whole sequences when the batch has more CSR rows than
  // the CSR passes hold (a caller's CSR covers the whole batch, so it must fit)
  const long long nrows = static_cast<long long>(B) * nblk;
  const int bc = kv_sub_batch(B, nblk);
  if (bc == 0)
    return fail(MSA_ERR_NOT_SUPPORTED, "kv-centric path: Skv/128 = %d exceeds %d", nblk,
                kMaxCsrRows);
  if (have_csr && nrows > kMaxCsrRows)
    return fail(MSA_ERR_NOT_SUPPORTED, "prebuilt CSR: B*Skv/128 = %lld exceeds %d", nrows,
                kMaxCsrRows);
  const size_t need = kv_layout(static_cast<long long>(bc) * Sq, static_cast<long long>(bc) * nblk,
                                Hq, Hkv, topk).total;
  if (!workspace || workspace_bytes < need)
    return fail(MSA_ERR_INVALID_VALUE, "workspace too small: need %zu bytes, got %zu", need,
                workspace ? workspace_bytes : static_cast<size_t>(0));
  if (!aligned(workspace, 256)) return fail(MSA_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  const size_t kv_elem = kv_fp8 ? 1 : 2;
  for (int b0 = 0; b0 < B; b0 += bc) {
    const int nb = std::min(bc, B - b0);
    const long long q_off = static_cast<long long>(b0) * Sq * Hq * D;  // elements
    const long long kv_off = static_cast<long long>(b0) * Skv * Hkv * D;
    const long long l_off = static_cast<long long>(b0) * Hq * Sq;
    const KvLayout L = kv_layout(static_cast<long long>(nb) * Sq, static_cast<long long>(nb) * nblk,
                                 Hq, Hkv, topk);
    KvParams p{};
    p.q = static_cast<const uint16_t*>(q) + q_off;
    p.k = static_cast<const char*>(k) + kv_off * kv_elem;
    p.v = static_cast<const char*>(v) + kv_off * kv_elem;
    p.kv_fp8 = kv_fp8;
    p.B = nb; p.Sq = Sq; p.Skv = Skv; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk; p.topk = topk;
    p.nblk = nblk; p.nrows = nb * nblk;
    p.cap = static_cast<long long>(nb) * Sq * topk;
    p.causal = causal ? 1 : 0;
    p.scale_log2 = scale * kLog2e;
    p.inv_temp = inv_temp;
    rc = run_kvcentric(p, q2k + static_cast<long long>(b0) * Hkv * Sq * topk,
                       have_csr ? csr_row_ptr : nullptr, csr_q_idx, csr_slot, L,
                       static_cast<char*>(workspace), nullptr, static_cast<uint16_t*>(o) + q_off,
                       lse + l_off, lse_temperature ? lse_temperature + l_off : nullptr, st);
    if (rc) return rc;
  }
  return MSA_OK;
}

size_t msa_build_k2q_csr_workspace_size(int B, int Hkv, int Sq, int topk, int num_kv_blocks) {
  if (B <= 0 || Hkv <= 0 || Sq <= 0 || topk <= 0 || num_kv_blocks <= 0) return 0;
  return csr_workspace_bytes(B, Hkv, Sq, topk, B * num_kv_blocks);
}

int msa_build_k2q_csr(const int32_t* q2k, int B, int Hkv, int Sq, int topk, int num_kv_blocks,
                      int32_t* row_ptr, int32_t* q_idx, int32_t* slot, void* workspace,
                      size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (B <= 0 || Hkv <= 0 || Sq <= 0 || topk <= 0 || num_kv_blocks <= 0)
    return fail(MSA_ERR_INVALID_VALUE, "B, Hkv, Sq, topk and num_kv_blocks must be positive");
  if (topk > kMaxTopk) return fail(MSA_ERR_NOT_SUPPORTED, "topk %d not supported (1..32)", topk);
  if (static_cast<long long>(B) * Sq * topk > 0x7FFFFFFFLL)
    return fail(MSA_ERR_INVALID_VALUE, "B*Sq*topk exceeds the int32 index range");
  const long long nrows = static_cast<long long>(B) * num_kv_blocks;
  if (nrows > kMaxCsrRows)
    return fail(MSA_ERR_NOT_SUPPORTED, "B*num_kv_blocks = %lld exceeds %d", nrows, kMaxCsrRows);
  if (!q2k || !row_ptr || !q_idx) return fail(MSA_ERR_INVALID_VALUE, "null pointer");
  if (!aligned(q2k, 4) || !aligned(row_ptr, 4) || !aligned(q_idx, 4) || (slot && !aligned(slot, 4)))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned int32 pointer");
  const size_t need = csr_workspace_bytes(B, Hkv, Sq, topk, static_cast<int>(nrows));
  if (!workspace || workspace_bytes < need)
    return fail(MSA_ERR_INVALID_VALUE, "workspace too small: need %zu bytes", need);
  if (!aligned(workspace, 256)) return fail(MSA_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  hipError_t e = launch_build_csr(q2k, B, Hkv, Sq, topk, num_kv_blocks, row_ptr, q_idx, slot,
                                  workspace, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "k2q CSR build");
}

// ---------------------------------------------------------------------------
// Variable-length batches
// ---------------------------------------------------------------------------
int msa_sparse_fwd_varlen_path(int B, int total_q, int total_k, int Hq, int Hkv, int topk,
                               int path) {
  (void)Hq;
  return resolve_varlen_path(path, B, total_q, total_k, Hkv, topk);
}

static bool varlen_sizes_ok(int B, int total_q, int total_k, int Hq, int Hkv, int D, int topk,
                            int blk_kv) {
  return B > 0 && total_q >= 0 && total_k >= 0 && Hq > 0 && Hkv > 0 && topk > 0 && D == kD &&
         blk_kv == kBlk && Hq % Hkv == 0;
}

size_t msa_sparse_fwd_varlen_workspace_size(int B, int total_q, int total_k, int Hq, int Hkv,
                                            int D, int topk, int blk_kv, int path) {
  if (!varlen_sizes_ok(B, total_q, total_k, Hq, Hkv, D, topk, blk_kv) || total_k == 0) return 0;
  if (resolve_varlen_path(path, B, total_q, total_k, Hkv, topk) != MSA_PATH_KVCENTRIC) return 0;
  const long long nrows = varlen_rows_bound(B, total_k);
  return align256(varlen_tables_bytes(B, total_q, nrows)) +
         kv_layout(total_q, nrows, Hq, Hkv, topk).total;
}

int msa_sparse_fwd_varlen(const void* q, const void* k, const void* v, const int32_t* q2k,
                          const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                          const int32_t* csr_row_ptr, const int32_t* csr_q_idx,
                          const int32_t* csr_slot, int csr_total_rows, int B, int total_q,
                          int total_k, int Hq, int Hkv, int D, int topk, int blk_kv, int causal,
                          float softmax_scale, int path, int kv_dtype, void* o, float* lse,
                          float lse_temperature_scale, float* lse_temperature, void* workspace,
                          size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (B <= 0 || total_q < 0 || total_k < 0)
    return fail(MSA_ERR_INVALID_VALUE, "B must be positive, total_q and total_k non-negative");
  int rc = check_common(B, 1, Hq, Hkv, D, topk, blk_kv);
  if (rc) return rc;
  rc = check_temperature(lse_temperature_scale, lse_temperature);
  if (rc) return rc;
  const float inv_temp = lse_temperature ? 1.f / lse_temperature_scale : 1.f;
  if (static_cast<long long>(total_q) * topk > 0x7FFFFFFFLL)
    return fail(MSA_ERR_INVALID_VALUE, "total_q*topk exceeds the int32 index range");
  if (path != MSA_PATH_AUTO && path != MSA_PATH_QCENTRIC && path != MSA_PATH_KVCENTRIC)
    return fail(path == MSA_PATH_TILE || path == MSA_PATH_DECODE ? MSA_ERR_NOT_SUPPORTED
                                                                 : MSA_ERR_INVALID_VALUE,
                "path %d not available for variable-length batches", path);
  if (!cu_seqlens_q || !cu_seqlens_k) return fail(MSA_ERR_INVALID_VALUE, "null cu_seqlens pointer");
  if (!aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned cu_seqlens pointer");
  const bool have_csr = csr_row_ptr || csr_q_idx || csr_slot;
  if (have_csr && !(csr_row_ptr && csr_q_idx && csr_slot))
    return fail(MSA_ERR_INVALID_VALUE, "csr_row_ptr, csr_q_idx and csr_slot go together");
  if (total_q == 0) return MSA_OK;  // nothing to compute or write
  if (!q || !q2k || !o || !lse || (total_k > 0 && (!k || !v)))
    return fail(MSA_ERR_INVALID_VALUE, "null tensor pointer");
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
      !aligned(q2k, 4) || !aligned(lse, 4))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned tensor pointer (bf16 tensors need 16 bytes)");
  const long long nrows_bound = varlen_rows_bound(B, total_k);
  if (have_csr && (csr_total_rows <= 0 || csr_total_rows > nrows_bound))
    return fail(MSA_ERR_INVALID_VALUE,
                "csr_total_rows (%d) must be in [1, floor(total_k / 128) + B = %lld]",
                csr_total_rows, nrows_bound);
  const int qpk = Hq / Hkv;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(D));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  int which = resolve_varlen_path(path, B, total_q, total_k, Hkv, topk);
  if (total_k == 0) which = MSA_PATH_QCENTRIC;  // no keys: every row is empty
  rc = check_kv_dtype(kv_dtype, which);
  if (rc) return rc;
  const int kv_fp8 = kv_dtype == MSA_DTYPE_FP8_E4M3;

  if (which == MSA_PATH_QCENTRIC) {
    QcParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = k;
    p.v = v;
    p.kv_fp8 = kv_fp8;
    p.q2k = q2k;
    p.cu_q = cu_seqlens_q;
    p.cu_k = cu_seqlens_k;
    p.total_q = total_q;
    p.total_k = total_k;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk; p.topk = topk;
    p.causal = causal ? 1 : 0;
    p.kv_stream = static_cast<long long>(total_q) *
                      std::min<long long>(topk, (total_k + kBlk - 1) / kBlk) <
                  kKvMinEntriesPerRow * varlen_rows_bound(B, total_k);
    p.scale_log2 = scale * kLog2e;
    p.splits = 1;
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.inv_temp = inv_temp;
    p.lse_t = lse_temperature;
    prof_mark(g_prof_before, st);
    hipError_t e = launch_qcentric(p, false, st);
    prof_mark(g_prof_after, st);
    return e == hipSuccess ? MSA_OK : hip_fail(e, "q-centric varlen forward");
  }

  // kv-centric
  if (nrows_bound > kMaxCsrRows)
    return fail(MSA_ERR_NOT_SUPPORTED,
                "kv-centric path: floor(total_k/128) + B = %lld CSR rows exceed %d", nrows_bound,
                kMaxCsrRows);
  const long long nrows = have_csr ? csr_total_rows : nrows_bound;
  const size_t tbytes = align256(varlen_tables_bytes(B, total_q, nrows_bound));
  const KvLayout L = kv_layout(total_q, nrows_bound, Hq, Hkv, topk);
  if (!workspace || workspace_bytes < tbytes + L.total)
    return fail(MSA_ERR_INVALID_VALUE, "workspace too small: need %zu bytes, got %zu",
                tbytes + L.total, workspace ? workspace_bytes : static_cast<size_t>(0));
  if (!aligned(workspace, 256)) return fail(MSA_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const VarlenTables vt = varlen_tables_at(ws, B, total_q, nrows);
  hipError_t e = launch_varlen_tables(cu_seqlens_q, cu_seqlens_k, B, total_q, total_k, nrows, vt, st);
  if (e != hipSuccess) return hip_fail(e, "varlen tables");
  KvParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = k;
  p.v = v;
  p.kv_fp8 = kv_fp8;
  p.B = 1; p.Sq = total_q; p.Skv = 0; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk; p.topk = topk;
  p.nblk = 0; p.nrows = static_cast<int>(nrows);
  p.cap = static_cast<long long>(total_q) * topk;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.total_q = total_q;
  p.total_k = total_k;
  p.inv_temp = inv_temp;
  return run_kvcentric(p, q2k, have_csr ? csr_row_ptr : nullptr, csr_q_idx, csr_slot, L,
                       ws + tbytes, &vt, static_cast<uint16_t*>(o), lse, lse_temperature, st);
}

size_t msa_build_k2q_csr_varlen_workspace_size(int B, int Hkv, int total_q, int topk,
                                               int total_rows) {
  if (B <= 0 || Hkv <= 0 || total_q <= 0 || topk <= 0 || total_rows <= 0) return 0;
  return align256(varlen_tables_bytes(B, total_q, 0)) +
         csr_workspace_bytes(1, Hkv, total_q, topk, total_rows);
}

int msa_build_k2q_csr_varlen(const int32_t* q2k, const int32_t* cu_seqlens_q,
                             const int32_t* cu_seqlens_k, int B, int Hkv, int total_q, int total_k,
                             int topk, int total_rows, int32_t* row_ptr, int32_t* q_idx,
                             int32_t* slot, void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (B <= 0 || Hkv <= 0 || total_q <= 0 || total_k < 0 || topk <= 0 || total_rows <= 0)
    return fail(MSA_ERR_INVALID_VALUE,
                "B, Hkv, total_q, topk and total_rows must be positive, total_k non-negative");
  if (topk > kMaxTopk) return fail(MSA_ERR_NOT_SUPPORTED, "topk %d not supported (1..32)", topk);
  if (static_cast<long long>(total_q) * topk > 0x7FFFFFFFLL)
    return fail(MSA_ERR_INVALID_VALUE, "total_q*topk exceeds the int32 index range");
  if (total_rows > kMaxCsrRows)
    return fail(MSA_ERR_NOT_SUPPORTED, "total_rows = %d exceeds %d", total_rows, kMaxCsrRows);
  if (!q2k || !cu_seqlens_q || !cu_seqlens_k || !row_ptr || !q_idx)
    return fail(MSA_ERR_INVALID_VALUE, "null pointer");
  if (!aligned(q2k, 4) || !aligned(cu_seqlens_q, 4) || !aligned(cu_seqlens_k, 4) ||
      !aligned(row_ptr, 4) || !aligned(q_idx, 4) || (slot && !aligned(slot, 4)))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned int32 pointer");
  const size_t tbytes = align256(varlen_tables_bytes(B, total_q, 0));
  const size_t need = tbytes + csr_workspace_bytes(1, Hkv, total_q, topk, total_rows);
  if (!workspace || workspace_bytes < need)
    return fail(MSA_ERR_INVALID_VALUE, "workspace too small: need %zu bytes", need);
  if (!aligned(workspace, 256)) return fail(MSA_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* ws = static_cast<char*>(workspace);
  const VarlenTables vt = varlen_tables_at(ws, B, total_q, 0);
  hipError_t e = launch_varlen_tables(cu_seqlens_q, cu_seqlens_k, B, total_q, total_k, 0, vt, st);
  if (e != hipSuccess) return hip_fail(e, "varlen tables");
  e = launch_build_csr_varlen(q2k, vt, Hkv, total_q, topk, total_rows, row_ptr, q_idx, slot,
                              ws + tbytes, st);
  return e == hipSuccess ? MSA_OK : hip_fail(e, "k2q CSR build (varlen)");
}

// ---------------------------------------------------------------------------
// Dense paged decode: plan / run
// ---------------------------------------------------------------------------
int msa_paged_decode_plan_init(int B, int Sq, int Hq, int Hkv, int D, int page_size,
                               int max_seqlen_k, int max_grid_size, int fixed_split_pages,
                               int disable_split_kv, msa_decode_plan* plan) {
  g_last_error.clear();
  if (!plan) return fail(MSA_ERR_INVALID_VALUE, "null plan");
  int rc = check_common(B, Sq, Hq, Hkv, D, 1, page_size);
  if (rc) return rc;
  if (Sq > 4 * kMaxQPerWave)
    return fail(MSA_ERR_NOT_SUPPORTED, "dense decode needs Sq <= %d (got %d)", 4 * kMaxQPerWave, Sq);
  if (max_seqlen_k <= 0) return fail(MSA_ERR_INVALID_VALUE, "max_seqlen_k must be positive");
  if (max_grid_size < 0 || fixed_split_pages < 0)
    return fail(MSA_ERR_INVALID_VALUE, "max_grid_size and fixed_split_pages must be >= 0");
  const int max_pages = (max_seqlen_k + kBlk - 1) / kBlk;
  int chunk;
  if (fixed_split_pages > 0) {
    if (fixed_split_pages > kDecMaxEntries)
      return fail(MSA_ERR_NOT_SUPPORTED, "fixed_split_pages %d exceeds %d", fixed_split_pages,
                  kDecMaxEntries);
    chunk = fixed_split_pages;
  } else if (disable_split_kv) {
    if (max_pages > kDecMaxEntries)
      return fail(MSA_ERR_NOT_SUPPORTED,
                  "disable_split_kv needs max_seqlen_k <= %d tokens (one chunk per sequence)",
                  kDecMaxEntries * kBlk);
    chunk = max_pages;
  } else {
    // aim at max_grid (sequence, chunk, KV head) items: split only when the
    // sequences alone leave the grid short
    const long long target = max_grid_size > 0 ? max_grid_size : 2LL * device_cu_count();
    const long long units = static_cast<long long>(B) * Hkv;
    const long long want = units >= target ? 1 : (target + units - 1) / units;
    chunk = static_cast<int>((max_pages + want - 1) / want);
    chunk = std::max(1, std::min(chunk, kDecMaxEntries));
  }
  const int max_chunks = (max_pages + chunk - 1) / chunk;
  msa_decode_plan P{};
  P.batch = B; P.seqlen_q = Sq; P.num_qo_heads = Hq; P.num_kv_heads = Hkv; P.max_pages = max_pages;
  P.kv_chunk_size_pages = chunk;
  P.split_kv = max_chunks > 1 ? 1 : 0;
  const long long padded = static_cast<long long>(B) * max_chunks;
  if (padded * Hkv > 0x7FFFFFFFLL) return fail(MSA_ERR_INVALID_VALUE, "problem too large");
  P.padded_work_count = static_cast<int>(padded);
  P.partial_rows = static_cast<int64_t>(padded) * Sq;
  size_t off = 0;
  P.kv_pages = off; off += align256(static_cast<size_t>(B) * 4);
  P.split_counts = off; off += align256(static_cast<size_t>(B) * 4);
  P.o_indptr = off; off += align256((static_cast<size_t>(B) + 1) * 4);
  P.merge_indptr = off; off += align256((static_cast<size_t>(B) * Sq + 1) * 4);
  P.work_offsets = off; off += align256(static_cast<size_t>(B) * 4);
  P.work_items = off; off += align256(static_cast<size_t>(padded) * 16);
  P.work_count = off; off += 256;
  const size_t prow = P.split_kv ? static_cast<size_t>(P.partial_rows) * Hq : 0;
  P.o_partial = off; off += align256(prow * kD * 4);
  P.lse_partial = off; off += align256(prow * 4);
  P.lse_t_partial = off; off += align256(prow * 4);
  P.bytes = off;
  *plan = P;
  return MSA_OK;
}

static int check_plan_buffer(const msa_decode_plan* plan, const void* buffer, size_t bytes) {
  if (!plan || !buffer) return fail(MSA_ERR_INVALID_VALUE, "null plan or plan buffer");
  if (plan->batch <= 0 || plan->seqlen_q <= 0 || plan->kv_chunk_size_pages <= 0 ||
      plan->kv_chunk_size_pages > kDecMaxEntries || plan->padded_work_count <= 0)
    return fail(MSA_ERR_INVALID_VALUE, "plan not initialised by msa_paged_decode_plan_init");
  if (bytes < plan->bytes)
    return fail(MSA_ERR_INVALID_VALUE, "plan buffer too small: need %zu bytes", plan->bytes);
  if (!aligned(buffer, 256)) return fail(MSA_ERR_INVALID_VALUE, "plan buffer must be 256-byte aligned");
  return MSA_OK;
}

static DecodeSchedule schedule_at(const msa_decode_plan* plan, void* buffer) {
  char* b = static_cast<char*>(buffer);
  DecodeSchedule s;
  s.kv_pages = reinterpret_cast<int32_t*>(b + plan->kv_pages);
  s.counts = reinterpret_cast<int32_t*>(b + plan->split_counts);
  s.o_indptr = reinterpret_cast<int32_t*>(b + plan->o_indptr);
  s.merge_indptr = reinterpret_cast<int32_t*>(b + plan->merge_indptr);
  s.work_off = reinterpret_cast<int32_t*>(b + plan->work_offsets);
  s.items = reinterpret_cast<int4*>(b + plan->work_items);
  s.work_count = reinterpret_cast<int32_t*>(b + plan->work_count);
  return s;
}

int msa_paged_decode_plan(const int32_t* seqused_k, const msa_decode_plan* plan, void* buffer,
                          size_t buffer_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_plan_buffer(plan, buffer, buffer_bytes);
  if (rc) return rc;
  if (!seqused_k || !aligned(seqused_k, 4)) return fail(MSA_ERR_INVALID_VALUE, "bad seqused_k pointer");
  const hipError_t e =
      launch_decode_schedule(seqused_k, plan->batch, plan->seqlen_q, plan->max_pages,
                             plan->kv_chunk_size_pages, plan->split_kv != 0,
                             schedule_at(plan, buffer), static_cast<hipStream_t>(stream));
  return e == hipSuccess ? MSA_OK : hip_fail(e, "decode schedule");
}

int msa_paged_decode_run(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, const int32_t* seqused_k,
                         const msa_decode_plan* plan, void* buffer, size_t buffer_bytes,
                         int num_pages, int dtype, int causal, float softmax_scale, void* o,
                         float* lse, float lse_temperature_scale, float* lse_temperature,
                         void* stream) {
  g_last_error.clear();
  int rc = check_plan_buffer(plan, buffer, buffer_bytes);
  if (rc) return rc;
  rc = check_temperature(lse_temperature_scale, lse_temperature);
  if (rc) return rc;
  rc = check_kv_dtype(dtype, MSA_PATH_AUTO);
  if (rc) return rc;
  if (dtype == MSA_DTYPE_FP8_E4M3 &&
      plan->seqlen_q * (plan->num_qo_heads / plan->num_kv_heads) > 128)
    return fail(MSA_ERR_NOT_SUPPORTED,
                "the fp8 dense decode needs Sq * Hq / Hkv <= 128 (got %d * %d)", plan->seqlen_q,
                plan->num_qo_heads / plan->num_kv_heads);
  if (num_pages <= 0) return fail(MSA_ERR_INVALID_VALUE, "num_pages must be positive");
  if (!q || !k_pool || !v_pool || !page_table || !seqused_k || !o || !lse)
    return fail(MSA_ERR_INVALID_VALUE, "null tensor pointer");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
      !aligned(lse, 4) || !aligned(page_table, 4) || !aligned(seqused_k, 4))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned tensor pointer (bf16 tensors need 16 bytes)");
  const msa_decode_plan& P = *plan;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(kD));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const DecodeSchedule S = schedule_at(plan, buffer);
  char* b = static_cast<char*>(buffer);
  QcParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = k_pool;
  p.v = v_pool;
  p.kv_fp8 = dtype == MSA_DTYPE_FP8_E4M3 ? 1 : 0;  // Q too: the pages' fp8 decode
  p.page_table = page_table;
  p.seqused = seqused_k;
  p.B = P.batch; p.Sq = P.seqlen_q; p.Hq = P.num_qo_heads; p.Hkv = P.num_kv_heads;
  p.qpk = P.num_qo_heads / P.num_kv_heads;
  p.max_pages = P.max_pages; p.num_pages = num_pages; p.nblk = P.max_pages;
  p.Skv = P.max_pages * kBlk;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;
  p.splits = 1;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.inv_temp = lse_temperature ? 1.f / lse_temperature_scale : 1.f;
  p.lse_t = lse_temperature;
  p.o_part = reinterpret_cast<float*>(b + P.o_partial);
  p.lse_part = reinterpret_cast<float*>(b + P.lse_partial);
  p.lse_t_part = lse_temperature ? reinterpret_cast<float*>(b + P.lse_t_partial) : nullptr;
  p.dec_items = S.items;
  p.dec_counts = S.counts;
  p.dec_o_indptr = S.o_indptr;
  p.dec_work_count = S.work_count;
  prof_mark(g_prof_before, st);
  hipError_t e = launch_dense_decode(p, P.padded_work_count, st);
  prof_mark(g_prof_after, st);
  if (e != hipSuccess) return hip_fail(e, "dense decode");
  if (P.split_kv) {
    e = launch_merge_decode(p.o_part, p.lse_part, p.lse_t_part, S.counts, S.o_indptr, P.batch,
                            P.seqlen_q, P.num_qo_heads, static_cast<uint16_t*>(o), lse,
                            lse_temperature, st);
    if (e != hipSuccess) return hip_fail(e, "decode merge");
  }
  return MSA_OK;
}

int msa_paged_sparse_fwd_path(int B, int Sq, int Hkv, int topk, int max_pages, int path) {
  if (path != MSA_PATH_AUTO) return path;
  if (B <= 0 || Sq <= 0 || Hkv <= 0 || topk <= 0 || max_pages <= 0) return MSA_PATH_QCENTRIC;
  return paged_plan(B, Sq, Hkv, topk, max_pages, 0, path).path;
}

int msa_paged_sparse_fwd_splits(int B, int Sq, int Hkv, int topk, int max_pages, int num_splits,
                                int path) {
  if (B <= 0 || Sq <= 0 || Hkv <= 0 || topk <= 0 || max_pages <= 0 || num_splits < 0) return 0;
  return paged_plan(B, Sq, Hkv, topk, max_pages, num_splits, path).splits;
}

size_t msa_paged_sparse_fwd_workspace_size(int B, int Sq, int Hq, int Hkv, int D, int topk,
                                           int page_size, int max_pages, int num_splits,
                                           int path) {
  if (B <= 0 || Sq <= 0 || Hq <= 0 || Hkv <= 0 || topk <= 0 || D != kD || page_size != kBlk ||
      max_pages <= 0 || Hq % Hkv || num_splits < 0)
    return 0;
  if (path != MSA_PATH_AUTO && path != MSA_PATH_QCENTRIC && path != MSA_PATH_DECODE &&
      path != MSA_PATH_KVCENTRIC)
    return 0;
  return paged_workspace(B, Sq, Hq, Hkv, topk, max_pages,
                         paged_plan(B, Sq, Hkv, topk, max_pages, num_splits, path));
}

int msa_paged_sparse_fwd(const void* q, const void* k_pool, const void* v_pool,
                         const int32_t* page_table, const int32_t* seqused_k, const int32_t* q2k,
                         int B, int Sq, int Hq, int Hkv, int D, int topk, int page_size,
                         int num_pages, int max_pages, int causal, float softmax_scale,
                         int num_splits, int path, int kv_dtype, void* o, float* lse,
                         float lse_temperature_scale, float* lse_temperature, void* workspace,
                         size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  int rc = check_common(B, Sq, Hq, Hkv, D, topk, page_size);
  if (rc) return rc;
  rc = check_temperature(lse_temperature_scale, lse_temperature);
  if (rc) return rc;
  if (num_pages <= 0 || max_pages <= 0)
    return fail(MSA_ERR_INVALID_VALUE, "num_pages and max_pages must be positive");
  if (!q || !k_pool || !v_pool || !page_table || !seqused_k || !q2k || !o || !lse)
    return fail(MSA_ERR_INVALID_VALUE, "null tensor pointer");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
      !aligned(q2k, 4) || !aligned(lse, 4) || !aligned(page_table, 4) || !aligned(seqused_k, 4))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned tensor pointer (bf16 tensors need 16 bytes)");
  if (num_splits < 0) return fail(MSA_ERR_INVALID_VALUE, "num_splits must be >= 0");
  if (path != MSA_PATH_AUTO && path != MSA_PATH_QCENTRIC && path != MSA_PATH_DECODE &&
      path != MSA_PATH_KVCENTRIC)
    return fail(MSA_ERR_INVALID_VALUE, "unknown paged path %d", path);
  if (path == MSA_PATH_DECODE && !paged_decode_supported(Sq, topk))
    return fail(MSA_ERR_NOT_SUPPORTED,
                "decode path needs Sq <= %d and Sq * topk <= %d (got Sq %d, topk %d)",
                4 * kMaxQPerWave, kDecMaxEntries, Sq, topk);
  const PagedPlan plan = paged_plan(B, Sq, Hkv, topk, max_pages, num_splits, path);
  const int splits = plan.splits;
  rc = check_kv_dtype(kv_dtype, plan.path);
  if (rc) return rc;
  const int qpk = Hq / Hkv;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(D));
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const float inv_temp = lse_temperature ? 1.f / lse_temperature_scale : 1.f;

  if (plan.path == MSA_PATH_KVCENTRIC) {
    // the contiguous kv-centric pipeline over max_pages blocks per sequence, each block
    // read through the page table; sub-batches of whole sequences past the CSR limit
    const int bc = kv_sub_batch(B, max_pages);
    if (bc == 0)
      return fail(MSA_ERR_NOT_SUPPORTED, "kv-centric path: max_pages = %d exceeds %d", max_pages,
                  kMaxCsrRows);
    const size_t need = paged_workspace(B, Sq, Hq, Hkv, topk, max_pages, plan);
    if (!workspace || workspace_bytes < need)
      return fail(MSA_ERR_INVALID_VALUE, "workspace too small: need %zu bytes, got %zu", need,
                  workspace ? workspace_bytes : static_cast<size_t>(0));
    if (!aligned(workspace, 256))
      return fail(MSA_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
    for (int b0 = 0; b0 < B; b0 += bc) {
      const int nb = std::min(bc, B - b0);
      const long long q_off = static_cast<long long>(b0) * Sq * Hq * D;  // elements
      const long long l_off = static_cast<long long>(b0) * Hq * Sq;
      const KvLayout L = kv_layout(static_cast<long long>(nb) * Sq,
                                   static_cast<long long>(nb) * max_pages, Hq, Hkv, topk);
      KvParams p{};
      p.q = static_cast<const uint16_t*>(q) + q_off;
      p.k = k_pool;
      p.v = v_pool;
      p.kv_fp8 = kv_dtype == MSA_DTYPE_FP8_E4M3;
      p.B = nb; p.Sq = Sq; p.Skv = max_pages * kBlk; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk;
      p.topk = topk; p.nblk = max_pages; p.nrows = nb * max_pages;
      p.cap = static_cast<long long>(nb) * Sq * topk;
      p.causal = causal ? 1 : 0;
      p.scale_log2 = scale * kLog2e;
      p.inv_temp = inv_temp;
      p.page_table = page_table + static_cast<long long>(b0) * max_pages;
      p.seqused = seqused_k + b0;
      p.num_pages = num_pages;
      rc = run_kvcentric(p, q2k + static_cast<long long>(b0) * Hkv * Sq * topk, nullptr, nullptr,
                         nullptr, L, static_cast<char*>(workspace), nullptr,
                         static_cast<uint16_t*>(o) + q_off, lse + l_off,
                         lse_temperature ? lse_temperature + l_off : nullptr, st);
      if (rc) return rc;
    }
    return MSA_OK;
  }

  QcParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = k_pool;
  p.v = v_pool;
  p.kv_fp8 = kv_dtype == MSA_DTYPE_FP8_E4M3;
  p.q2k = q2k;
  p.page_table = page_table;
  p.seqused = seqused_k;
  p.B = B; p.Sq = Sq; p.Skv = max_pages * kBlk; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk; p.topk = topk;
  p.nblk = max_pages; p.max_pages = max_pages; p.num_pages = num_pages;
  // fewer than two (query, slot) entries per block on average: each block is read about
  // once per (b, hkv), so its loads bypass the cache's retention
  p.kv_stream = static_cast<long long>(Sq) * std::min(topk, max_pages) <
                kKvMinEntriesPerRow * max_pages;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;
  p.splits = splits;
  p.o = static_cast<uint16_t*>(o);
  p.lse = lse;
  p.inv_temp = inv_temp;
  p.lse_t = lse_temperature;
  if (splits > 1) {
    const size_t need = paged_workspace(B, Sq, Hq, Hkv, topk, max_pages, plan);
    if (!workspace || workspace_bytes < need)
      return fail(MSA_ERR_INVALID_VALUE, "workspace too small: need %zu bytes", need);
    if (!aligned(workspace, 256)) return fail(MSA_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
    const size_t rows = static_cast<size_t>(B) * Sq * Hq;
    p.o_part = static_cast<float*>(workspace);
    char* wsc = static_cast<char*>(workspace);
    p.lse_part = reinterpret_cast<float*>(wsc + align256(splits * rows * kD * 4));
    if (lse_temperature)
      p.lse_t_part = reinterpret_cast<float*>(wsc + align256(splits * rows * kD * 4) +
                                              align256(splits * rows * 4));
  }
  prof_mark(g_prof_before, st);
  hipError_t e = plan.path == MSA_PATH_DECODE ? launch_paged_decode(p, st)
                                              : launch_qcentric(p, true, st);
  prof_mark(g_prof_after, st);
  if (e != hipSuccess) return hip_fail(e, "paged forward");
  if (splits > 1) {
    e = launch_combine_splits(p.o_part, p.lse_part, B, Sq, Hq, splits, static_cast<uint16_t*>(o),
                              lse, st, p.lse_t_part, lse_temperature);
    if (e != hipSuccess) return hip_fail(e, "split combine");
  }
  return MSA_OK;
}


// Paged K/V with a packed (variable-length) query batch: the paged form of
// sparse_atten_func with cu_seqlens_q. Sequence b owns max_pages CSR rows.
int msa_paged_sparse_fwd_varlen_path(int B, int total_q, int Hkv, int topk, int max_pages,
                                     int path) {
  if (path != MSA_PATH_AUTO) return path;
  if (B <= 0 || total_q <= 0 || Hkv <= 0 || topk <= 0 || max_pages <= 0) return MSA_PATH_QCENTRIC;
  const long long nrows = static_cast<long long>(B) * max_pages;
  return nrows <= kMaxCsrRows && kv_pays(total_q, Hkv, topk, max_pages, nrows)
             ? MSA_PATH_KVCENTRIC
             : MSA_PATH_QCENTRIC;
}

// q-centric splits of a paged varlen batch: the uniform paged rule with total_q query rows
int paged_varlen_splits(int total_q, int Hkv, int topk, int num_splits) {
  return qcentric_splits(static_cast<long long>(total_q) * Hkv, topk, num_splits);
}

int msa_paged_sparse_fwd_varlen_splits(int B, int total_q, int Hkv, int topk, int max_pages,
                                       int num_splits, int path) {
  if (B <= 0 || total_q <= 0 || Hkv <= 0 || topk <= 0 || max_pages <= 0 || num_splits < 0)
    return 0;
  if (msa_paged_sparse_fwd_varlen_path(B, total_q, Hkv, topk, max_pages, path) !=
      MSA_PATH_QCENTRIC)
    return 1;
  return paged_varlen_splits(total_q, Hkv, topk, num_splits);
}

size_t msa_paged_sparse_fwd_varlen_workspace_size(int B, int total_q, int Hq, int Hkv, int D,
                                                  int topk, int page_size, int max_pages,
                                                  int num_splits, int path) {
  if (B <= 0 || total_q <= 0 || Hq <= 0 || Hkv <= 0 || topk <= 0 || D != kD ||
      page_size != kBlk || max_pages <= 0 || Hq % Hkv || num_splits < 0)
    return 0;
  if (msa_paged_sparse_fwd_varlen_path(B, total_q, Hkv, topk, max_pages, path) !=
      MSA_PATH_KVCENTRIC)
    return paged_workspace(total_q, 1, Hq, Hkv, topk, max_pages,
                           PagedPlan{MSA_PATH_QCENTRIC,
                                     paged_varlen_splits(total_q, Hkv, topk, num_splits)});
  const long long nrows = static_cast<long long>(B) * max_pages;
  if (nrows > kMaxCsrRows) return 0;
  return align256(varlen_tables_bytes(B, total_q, nrows)) +
         kv_layout(total_q, nrows, Hq, Hkv, topk).total;
}

int msa_paged_sparse_fwd_varlen(const void* q, const void* k_pool, const void* v_pool,
                                const int32_t* page_table, const int32_t* seqused_k,
                                const int32_t* cu_seqlens_q, const int32_t* q2k, int B,
                                int total_q, int Hq, int Hkv, int D, int topk, int page_size,
                                int num_pages, int max_pages, int causal, float softmax_scale,
                                int num_splits, int path, int kv_dtype, void* o, float* lse,
                                float lse_temperature_scale, float* lse_temperature,
                                void* workspace, size_t workspace_bytes, void* stream) {
  g_last_error.clear();
  if (num_splits < 0) return fail(MSA_ERR_INVALID_VALUE, "num_splits must be >= 0");
  if (B <= 0 || total_q < 0)
    return fail(MSA_ERR_INVALID_VALUE, "B must be positive and total_q non-negative");
  int rc = check_common(B, 1, Hq, Hkv, D, topk, page_size);
  if (rc) return rc;
  rc = check_temperature(lse_temperature_scale, lse_temperature);
  if (rc) return rc;
  if (static_cast<long long>(total_q) * topk > 0x7FFFFFFFLL)
    return fail(MSA_ERR_INVALID_VALUE, "total_q*topk exceeds the int32 index range");
  if (num_pages <= 0 || max_pages <= 0)
    return fail(MSA_ERR_INVALID_VALUE, "num_pages and max_pages must be positive");
  if (path != MSA_PATH_AUTO && path != MSA_PATH_QCENTRIC && path != MSA_PATH_KVCENTRIC)
    return fail(path == MSA_PATH_TILE || path == MSA_PATH_DECODE ? MSA_ERR_NOT_SUPPORTED
                                                                 : MSA_ERR_INVALID_VALUE,
                "path %d not available for variable-length paged batches", path);
  if (!cu_seqlens_q || !page_table || !seqused_k)
    return fail(MSA_ERR_INVALID_VALUE, "null pointer");
  if (!aligned(cu_seqlens_q, 4) || !aligned(page_table, 4) || !aligned(seqused_k, 4))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned int32 pointer");
  if (total_q == 0) return MSA_OK;  // nothing to compute or write
  if (!q || !k_pool || !v_pool || !q2k || !o || !lse)
    return fail(MSA_ERR_INVALID_VALUE, "null tensor pointer");
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(o, 16) ||
      !aligned(q2k, 4) || !aligned(lse, 4))
    return fail(MSA_ERR_INVALID_VALUE, "misaligned tensor pointer (bf16 tensors need 16 bytes)");
  const int which = msa_paged_sparse_fwd_varlen_path(B, total_q, Hkv, topk, max_pages, path);
  rc = check_kv_dtype(kv_dtype, which);
  if (rc) return rc;
  const int qpk = Hq / Hkv;
  const int kv_fp8 = kv_dtype == MSA_DTYPE_FP8_E4M3;
  const float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf(static_cast<float>(D));
  const float inv_temp = lse_temperature ? 1.f / lse_temperature_scale : 1.f;
  const hipStream_t st = static_cast<hipStream_t>(stream);

  if (which == MSA_PATH_QCENTRIC) {
    QcParams p{};
    p.q = static_cast<const uint16_t*>(q);
    p.k = k_pool;
    p.v = v_pool;
    p.kv_fp8 = kv_fp8;
    p.q2k = q2k;
    p.page_table = page_table;
    p.seqused = seqused_k;
    p.cu_q = cu_seqlens_q;
    p.total_q = total_q;
    p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk; p.topk = topk;
    p.nblk = max_pages; p.max_pages = max_pages; p.num_pages = num_pages;
    p.kv_stream = static_cast<long long>(total_q) * std::min(topk, max_pages) <
                  kKvMinEntriesPerRow * B * static_cast<long long>(max_pages);
    p.causal = causal ? 1 : 0;
    p.scale_log2 = scale * kLog2e;
    p.splits = paged_varlen_splits(total_q, Hkv, topk, num_splits);
    p.o = static_cast<uint16_t*>(o);
    p.lse = lse;
    p.inv_temp = inv_temp;
    p.lse_t = lse_temperature;
    if (p.splits > 1) {  // partials over total_q rows: the uniform layout with B = total_q, Sq = 1
      const PagedPlan pl{MSA_PATH_QCENTRIC, p.splits};
      const size_t need = paged_workspace(total_q, 1, Hq, Hkv, topk, max_pages, pl);
      if (!workspace || workspace_bytes < need)
        return fail(MSA_ERR_INVALID_VALUE, "workspace too small: need %zu bytes", need);
      if (!aligned(workspace, 256))
        return fail(MSA_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
      const size_t rows = static_cast<size_t>(total_q) * Hq;
      char* wsc = static_cast<char*>(workspace);
      p.o_part = reinterpret_cast<float*>(wsc);
      p.lse_part = reinterpret_cast<float*>(wsc + align256(p.splits * rows * kD * 4));
      if (lse_temperature)
        p.lse_t_part = reinterpret_cast<float*>(wsc + align256(p.splits * rows * kD * 4) +
                                                align256(p.splits * rows * 4));
    }
    prof_mark(g_prof_before, st);
    hipError_t e = launch_qcentric(p, true, st);
    prof_mark(g_prof_after, st);
    if (e != hipSuccess) return hip_fail(e, "q-centric paged varlen forward");
    if (p.splits > 1) {
      // LSE [total_q, Hq] is the uniform [B, Hq, Sq] layout with B = total_q, Sq = 1
      e = launch_combine_splits(p.o_part, p.lse_part, total_q, 1, Hq, p.splits,
                                static_cast<uint16_t*>(o), lse, st, p.lse_t_part, lse_temperature);
      if (e != hipSuccess) return hip_fail(e, "split combine");
    }
    return MSA_OK;
  }

  // kv-centric: max_pages CSR rows per sequence, all held by the CSR passes at once
  const long long nrows = static_cast<long long>(B) * max_pages;
  if (nrows > kMaxCsrRows)
    return fail(MSA_ERR_NOT_SUPPORTED, "kv-centric path: B*max_pages = %lld CSR rows exceed %d",
                nrows, kMaxCsrRows);
  const size_t tbytes = align256(varlen_tables_bytes(B, total_q, nrows));
  const KvLayout L = kv_layout(total_q, nrows, Hq, Hkv, topk);
  if (!workspace || workspace_bytes < tbytes + L.total)
    return fail(MSA_ERR_INVALID_VALUE, "workspace too small: need %zu bytes, got %zu",
                tbytes + L.total, workspace ? workspace_bytes : static_cast<size_t>(0));
  if (!aligned(workspace, 256)) return fail(MSA_ERR_INVALID_VALUE, "workspace must be 256-byte aligned");
  char* ws = static_cast<char*>(workspace);
  const VarlenTables vt = varlen_tables_at(ws, B, total_q, nrows);
  hipError_t e = launch_varlen_tables(cu_seqlens_q, nullptr, B, total_q, 0, nrows, vt, st,
                                      max_pages);
  if (e != hipSuccess) return hip_fail(e, "varlen tables");
  KvParams p{};
  p.q = static_cast<const uint16_t*>(q);
  p.k = k_pool;
  p.v = v_pool;
  p.kv_fp8 = kv_fp8;
  p.B = 1; p.Sq = total_q; p.Skv = 0; p.Hq = Hq; p.Hkv = Hkv; p.qpk = qpk; p.topk = topk;
  p.nblk = max_pages; p.nrows = static_cast<int>(nrows);
  p.cap = static_cast<long long>(total_q) * topk;
  p.causal = causal ? 1 : 0;
  p.scale_log2 = scale * kLog2e;
  p.cu_q = cu_seqlens_q;
  p.total_q = total_q;
  p.inv_temp = inv_temp;
  p.page_table = page_table;
  p.seqused = seqused_k;
  p.num_pages = num_pages;
  return run_kvcentric(p, q2k, nullptr, nullptr, nullptr, L, ws + tbytes, &vt,
                       static_cast<uint16_t*>(o), lse, lse_temperature, st);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Paged sparse forward for callers that cannot allocate (msa_paged_sparse_fwd_noalloc):
// the split partials live in a file-scope device array of MSA_NOALLOC_SCRATCH_BYTES.
// Each GPU the library runs on holds its own copy until the process ends. On the host
// the name `scratch` is only a stand-in: the device address of each GPU's copy is
// looked up once per device with hipGetSymbolAddress, that device current, and kept.
// ---------------------------------------------------------------------------
namespace {

constexpr size_t kNoAllocScratchBytes = MSA_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};

// this device's scratch address (looked up on the first call for the device)
int scratch_for_device(int dev, void** out) {
  if (dev < 0 || dev >= kMaxScratchDevices)
    return fail(MSA_ERR_NOT_SUPPORTED, "device %d beyond the %d the scratch table keeps", dev,
                kMaxScratchDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e, "hipSetDevice");
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev) (void)hipSetDevice(cur);
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!ptr || !aligned(ptr, 256))
      return fail(MSA_ERR_HIP, "scratch array has no usable device address");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MSA_OK;
}

}  // namespace

extern "C" {

int msa_paged_sparse_fwd_noalloc(const void* q, const void* k_pool, const void* v_pool,
                                 const int32_t* page_table, const int32_t* seqused_k,
                                 const int32_t* q2k, int B, int Sq, int Hq, int Hkv, int D,
                                 int topk, int page_size, int num_pages, int max_pages, int causal,
                                 float softmax_scale, int num_splits, int path, int kv_dtype,
                                 void* o, float* lse, float lse_temperature_scale,
                                 float* lse_temperature, void* stream) {
  g_last_error.clear();
  // The automatic path never takes the kv-centric one here: its partials (a bf16 row per
  // (query, head, slot)) outgrow the scratch on the problems it is chosen for.
  if (path == MSA_PATH_AUTO && msa_paged_sparse_fwd_path(B, Sq, Hkv, topk, max_pages, path) ==
                                   MSA_PATH_KVCENTRIC)
    path = MSA_PATH_QCENTRIC;
  // The scratch this call needs is the workspace msa_paged_sparse_fwd would take (0 for
  // one split, and for argument errors, which msa_paged_sparse_fwd reports itself).
  const size_t need = msa_paged_sparse_fwd_workspace_size(B, Sq, Hq, Hkv, D, topk, page_size,
                                                          max_pages, num_splits, path);
  if (need > kNoAllocScratchBytes)
    return fail(MSA_ERR_INVALID_VALUE,
                "split partials need %zu bytes; the no-allocation entry point holds %zu "
                "(fewer splits, or msa_paged_sparse_fwd with a workspace)",
                need, kNoAllocScratchBytes);
  void* ws = nullptr;
  if (need > 0) {
    const hipStream_t st = static_cast<hipStream_t>(stream);
    int dev = -1;
    const hipError_t e = st ? hipStreamGetDevice(st, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "device of the stream");
    const int rc = scratch_for_device(dev, &ws);
    if (rc) return rc;
  }
  return msa_paged_sparse_fwd(q, k_pool, v_pool, page_table, seqused_k, q2k, B, Sq, Hq, Hkv, D,
                              topk, page_size, num_pages, max_pages, causal, softmax_scale,
                              num_splits, path, kv_dtype, o, lse, lse_temperature_scale,
                              lse_temperature, ws, need > 0 ? kNoAllocScratchBytes : 0, stream);
}

}  // extern "C"
