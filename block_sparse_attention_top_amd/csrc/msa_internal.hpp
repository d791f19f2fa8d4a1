// Internal declarations shared by the HIP translation units of libmsa.
// gfx950 (CDNA4) only: wave64, bf16 MFMA 16x16x32 / 32x32x16, ds_read_b64_tr_b16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kD = 128;      // head dim (the only one supported)
constexpr int kBlk = 128;    // KV block / page size
constexpr int kMaxTopk = 32;
constexpr int kMaxCsrRows = 16384;  // B * num_kv_blocks: the CSR passes keep one int per row in LDS
constexpr int kKvChunkRows = 2048;  // (query, head) rows per kv-centric work item
constexpr int kKvMaxEntries = 512;  // CSR entries per kv-centric work item (LDS bound)
// kv-centric item order: kKvStreams streams (one per XCD) of kKvBucketsPerStream keys
constexpr int kKvStreams = 8;
constexpr int kKvBucketsPerStream = 256;
constexpr int kKvKeys = kKvStreams * kKvBucketsPerStream;
constexpr int kDecMaxEntries = 512; // Sq * topk index entries per paged decode workgroup
constexpr int kDecPasses = kDecMaxEntries / 256;
constexpr int kMaxQPerWave = 4;     // query rows per wave in the paged decode kernel (Sq <= 16)
constexpr int kMaxDecodeSplits = 64;
constexpr int kTileMaxQ = 32;       // queries per workgroup in the query-tile kernel (qpk 8)
constexpr int kTileMaxEntries = 512;  // index entries (queries x topk) per query tile

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// fp32 -> bf16
// ---------------------------------------------------------------------------
// Two fp32 -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// LDS tiles of 128-dim bf16 rows (256 B of data per row), padded so that the
// address of (row, byte) is linear -- every fragment read is one lane base plus
// an immediate offset. The strides were chosen by measuring LDS bank-conflict
// cycles on gfx950 (64 banks of 4 bytes) for the two read patterns used:
//   K tiles: row stride 272 B (68 banks): the 16-byte fragment reads of 16
//            consecutive rows start 4 banks apart -> conflict free
//            (288 B costs 4 conflict cycles per read, 320 B costs 12).
//   V tiles: row stride 320 B (80 banks): the transposed 8-byte reads of
//            4 rows x 2 column bands per half wave land on 8 distinct 8-bank
//            groups -> conflict free (272 B and 288 B cost 6 and 2 cycles).
// ---------------------------------------------------------------------------
constexpr int kKStride = 272;
constexpr int kVStride = 320;
__device__ __forceinline__ int k_off(int r, int c16) { return r * kKStride + c16 * 16; }
__device__ __forceinline__ int v_off(int r, int c16) { return r * kVStride + c16 * 16; }

// ds_read_b64_tr_b16: within each 16-lane group, lane j receives element
// (j % 4) of the 8-byte words addressed by lanes 4*i + j/4, i = 0..3.
// With lane l' of a group addressing row k0 + l'/4, columns d0 + 4*(l'%4)..+3
// of a row-major tile, lane j receives column d0 + j of rows k0..k0+3.
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(lds_ptr));
}

__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }
__device__ __forceinline__ bf16x8 cat_tr(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// fp8 e4m3fn K/V cache: 16 fp8 bytes -> 16 bf16 values (exact; e4m3fn is a subset
// of bf16), with the gfx950 conversion v_cvt_scalef32_pk_bf16_fp8 at scale 1
// (two bytes per instruction, OCP e4m3fn, NaN codes to NaN). out[0] holds
// elements 0..7, out[1] elements 8..15.
template <bool HI>
__device__ __forceinline__ uint32_t fp8x2_to_bf16x2(uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, HI));
}
__device__ __forceinline__ void fp8x16_to_bf16x16(u32x4 in, u32x4 out[2]) {
  out[0] = u32x4{fp8x2_to_bf16x2<false>(in[0]), fp8x2_to_bf16x2<true>(in[0]),
                 fp8x2_to_bf16x2<false>(in[1]), fp8x2_to_bf16x2<true>(in[1])};
  out[1] = u32x4{fp8x2_to_bf16x2<false>(in[2]), fp8x2_to_bf16x2<true>(in[2]),
                 fp8x2_to_bf16x2<false>(in[3]), fp8x2_to_bf16x2<true>(in[3])};
}

constexpr float kLn2 = 0.693147180559945309417f;
constexpr float kLog2e = 1.442695040888963407359f;

// Query range of global query q among `buckets` equal ranges of nq queries:
// floor(q * buckets / nq), clamped to [0, buckets - 1], with the product in 64 bits
// (q * 256 leaves the int32 range once q reaches 2^23). Every kernel that buckets
// an item by its first query calls this one function, so that all of them agree.
__host__ __device__ __forceinline__ int query_bucket(long long q, long long nq, int buckets) {
  const long long b = q * buckets / nq;
  return static_cast<int>(b < 0 ? 0 : (b >= buckets ? buckets - 1 : b));
}

// ---------------------------------------------------------------------------
// Variable-length batches. cu_q / cu_k are prefix sums over the B sequences
// (cu[0] = 0, cu[B] = total); sequence b owns the packed query rows
// [cu_q[b], cu_q[b+1]) and key rows [cu_k[b], cu_k[b+1]). Offsets read from
// them are clamped into [0, total] so that malformed prefix sums give
// unspecified values but never an access outside the packed tensors.
// ---------------------------------------------------------------------------
// largest b in [0, n) with cu[b] <= g (binary search; n >= 1)
__device__ __forceinline__ int seq_search(const int32_t* cu, int n, long long g) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= g) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}
// first row and length of sequence b in a packed dimension of `total` rows
__device__ __forceinline__ void seq_range(const int32_t* cu, int b, long long total,
                                          long long& beg, long long& len) {
  long long a = cu[b], e = cu[b + 1];
  a = a < 0 ? 0 : (a > total ? total : a);
  e = e < a ? a : (e > total ? total : e);
  beg = a;
  len = e - a;
}

// Per-sequence tables of a varlen batch, built on the device (msa_varlen.hip):
//   rowbase [B+1]      first k2q CSR row of each sequence: prefix sum of ceil(Skv_b / 128)
//   q_rows  [total_q]  (rowbase[b], ceil(Skv_b / 128)) of the sequence b of each query
//   row_seq [nrows]    sequence of each CSR row, -1 past rowbase[B]
struct VarlenTables {
  int32_t* rowbase;
  int2* q_rows;
  int32_t* row_seq;
};
size_t varlen_tables_bytes(int B, long long total_q, long long nrows);
// carves the tables out of ws (varlen_tables_bytes(...) bytes, 256-byte aligned)
VarlenTables varlen_tables_at(void* ws, int B, long long total_q, long long nrows);
// cu_k == nullptr: every sequence has blocks_per_seq blocks (a paged batch's max_pages)
hipError_t launch_varlen_tables(const int32_t* cu_q, const int32_t* cu_k, int B, long long total_q,
                                long long total_k, long long nrows, const VarlenTables& t,
                                hipStream_t stream, int blocks_per_seq = 0);

// ---------------------------------------------------------------------------
// Launchers (each returns hipGetLastError() after its launches).
// ---------------------------------------------------------------------------
struct QcParams {
  const uint16_t* q;
  const void* k;             // contiguous [B,Skv,Hkv,D] or pool [num_pages,Hkv,128,D]
  const void* v;             // (bf16, or fp8 e4m3fn bytes when kv_fp8)
  int kv_fp8;
  const int32_t* q2k;        // [B,Hkv,Sq,topk]
  const int32_t* page_table; // paged only: [B,max_pages]
  const int32_t* seqused;    // paged only: [B]
  int B, Sq, Skv, Hq, Hkv, qpk, topk;
  int nblk;                  // valid block ids are [0, nblk)
  int max_pages, num_pages;
  int kv_stream;             // blocks are read about once (load them non-temporally)
  int causal;
  float scale_log2;          // softmax_scale * log2(e)
  int splits;                // 1 = write final O/LSE
  uint16_t* o;               // bf16 [B,Sq,Hq,D]
  float* lse;                // [B,Hq,Sq]
  float* o_part;             // [splits][B*Sq][Hq][D]
  float* lse_part;           // [splits][B*Sq][Hq]
  // temperature-scaled LSE (log-sum-exp of the scores divided by T), written when
  // lse_t != nullptr, in the layout of lse; partials [splits][B*Sq][Hq] when split
  float inv_temp;            // 1 / T
  float* lse_t;
  float* lse_t_part;
  // variable-length batch: cu_q != nullptr. Then q is [total_q,Hq,D], q2k
  // [Hkv,total_q,topk], o [total_q,Hq,D], lse [total_q,Hq]; B is the sequence count
  // and Sq is unused. Contiguous K/V: k/v [total_k,Hkv,D] by cu_k (Skv, nblk unused);
  // paged: the pools, page_table and seqused as above, split partials over total_q rows.
  const int32_t* cu_q;
  const int32_t* cu_k;
  long long total_q, total_k;
  // dense paged decode (every key of the sequence, split-KV by a device schedule):
  // work item w = (b, chunk, first page, pages) for w < *dec_work_count; chunk c of
  // sequence b (of dec_counts[b] chunks) writes partial rows o_indptr[b] + q * count + c
  // when count > 1, else the final O / LSE
  const int4* dec_items;
  const int32_t* dec_counts;
  const int32_t* dec_o_indptr;
  const int32_t* dec_work_count;
};
hipError_t launch_qcentric(const QcParams& p, bool paged, hipStream_t stream);
// paged decode over the union of the blocks of each (b, hkv): splits partition that
// union; needs Sq <= 4 * kMaxQPerWave and Sq * topk <= kDecMaxEntries
bool paged_decode_supported(int Sq, int topk);
hipError_t launch_paged_decode(const QcParams& p, hipStream_t stream);
// dense decode over a schedule: grid = padded_work * Hkv (items past the count exit)
hipError_t launch_dense_decode(const QcParams& p, int padded_work, hipStream_t stream);
// the schedule: per sequence the pages ceil(seqused / 128) (clamped to max_pages), the
// chunk count max(1, ceil(pages / chunk_pages)) (1 when !split), o_indptr (exclusive
// prefix of count * Sq), merge_indptr[b * Sq + q] = o_indptr[b] + q * count, the work
// items and their count
struct DecodeSchedule {
  int32_t* kv_pages;      // [B]
  int32_t* counts;        // [B]
  int32_t* o_indptr;      // [B+1]
  int32_t* merge_indptr;  // [B*Sq+1]
  int32_t* work_off;      // [B] first work item of each sequence
  int4* items;            // [padded work]
  int32_t* work_count;    // [1]
};
hipError_t launch_decode_schedule(const int32_t* seqused, int B, int Sq, int max_pages,
                                  int chunk_pages, bool split, const DecodeSchedule& s,
                                  hipStream_t stream);
// merge of the dense decode's partial rows (sequences with more than one chunk)
hipError_t launch_merge_decode(const float* o_part, const float* lse_part, const float* lse_t_part,
                               const int32_t* counts, const int32_t* o_indptr, int B, int Sq,
                               int Hq, uint16_t* o, float* lse, float* lse_t, hipStream_t stream);

// query-tile kernel (contiguous K/V): a workgroup per 256 / qpk consecutive
// queries of one (b, hkv), streaming the union of their selected blocks once
struct TileParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const int32_t* q2k;
  int B, Sq, Skv, Hq, Hkv, qpk, topk, nblk, causal;
  float scale_log2;
  uint16_t* o;
  float* lse;
  float inv_temp;  // temperature-scaled LSE into lse_t (layout of lse) when lse_t != nullptr
  float* lse_t;
  int ntiles;     // set by the launcher
  int xcd_pairs;  // set by the launcher: (b, hkv) pairs mapped onto XCD groups
};
bool tile_supported(int qpk, int topk);  // qpk 8 or 16, tile queries x topk <= 512
hipError_t launch_tile(TileParams p, hipStream_t stream);

struct KvParams {
  const uint16_t* q;
  const void* k;             // bf16, or fp8 e4m3fn bytes when kv_fp8
  const void* v;
  int kv_fp8;
  const int32_t* row_ptr;    // [Hkv, nrows+1]
  const int32_t* q_idx;      // [Hkv, cap]: the query of each entry, or (slot == nullptr)
                             // its index query * topk + slot into the index table
  const int32_t* slot;       // [Hkv, cap] or nullptr
  const int4* items;         // (hkv, row, first entry, entry count), in key order
  const int32_t* key_start;  // [kKvKeys + 1] first item of each key (the streams' bounds)
  int32_t* stream_next;      // [kKvStreams] items taken from each stream (zero on entry)
  int streams;               // streams the key range is cut into: 1, 2, 4 or 8
  int B, Sq, Skv, Hq, Hkv, qpk, topk, nblk, nrows;
  long long cap;             // B*Sq*topk
  int chunk_entries;         // CSR entries per work item
  int causal;
  float scale_log2;
  uint16_t* o_part;          // bf16 [B*Sq][topk][Hkv][16 dim chunks][qpk][8], unnormalised:
                             // sum_j e^(s_j - M) V_j
  float2* lse_part;          // [B*Sq][topk][Hq]: (LSE of the block, reference max M), natural log
  float inv_temp;            // 1 / T of the temperature-scaled LSE
  float* lse_t_part;         // [B*Sq][topk][Hq] temperature-scaled LSE of the block, or nullptr
  // variable-length batch: cu_q != nullptr, rows r of sequence row_seq[r] hold its
  // block r - rowbase[b]; B*Sq above reads total_q (cap = total_q * topk)
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* rowbase;
  const int32_t* row_seq;
  long long total_q, total_k;
  // paged K/V (page_table != nullptr): block s of sequence b is page page_table[b * nblk + s]
  // of the pools [num_pages, Hkv, 128, D], and the sequence's keys are [0, seqused[b]);
  // with packed queries (cu_q) the rows of sequence b are rowbase[b] .. + nblk
  const int32_t* page_table;
  const int32_t* seqused;
  int num_pages;
};
// persistent grid (two workgroups per compute unit, at most max_items) over the
// streams of the key-ordered item table
hipError_t launch_kvcentric(const KvParams& p, long long max_items, hipStream_t stream);
// The item order's counters: counts, next, bad and cursor must be zero before the item
// table is filled (the CSR count pass, or a fill kernel for a caller's CSR, clears the
// first kKvSortZeroInts ints, which hold all four).
struct KvSortBuffers {
  int32_t* counts;     // [kKvKeys] items per key
  int32_t* next;       // [kKvStreams] items taken from each stream (KvParams::stream_next)
  int32_t* bad;        // [1] set when a caller's CSR row_ptr is not non-decreasing in [0, cap]
  int32_t* cursor;     // [kKvKeys] items placed per key by the sort
  int32_t* key_start;  // [kKvKeys + 1] first item of each key (written by the sort)
};
// counts, next, bad and cursor lie in the first kKvSortZeroInts ints, which must be zero
// before the item table is built
static_assert(kKvStreams < 16, "next and bad share 16 ints");
constexpr int kKvSortZeroInts = kKvKeys + 16 + kKvKeys;
constexpr int kKvSortInts = kKvSortZeroInts + kKvKeys + 1;
inline KvSortBuffers kv_sort_buffers(int32_t* base) {
  return KvSortBuffers{base, base + kKvKeys, base + kKvKeys + kKvStreams, base + kKvKeys + 16,
                       base + kKvSortZeroInts};
}
// The unsorted item table has a fixed slot for every possible item: item j of row r
// of KV head hkv starts at row position p = row start + j * chunk, and
//   slot = hkv * per_head + floor(p / chunk) + r,  per_head = cap / chunk + nrows + 1,
// which grows strictly with (r, j) (a row's first chunk starts at or after its
// predecessor's last one) and stays below per_head. Unused slots hold entry count 0:
// the table is cleared (as ints) before it is filled.
__host__ __device__ inline long long kv_item_slot(int hkv, long long per_head, int pos,
                                                  int chunk_shift, int row) {
  return static_cast<long long>(hkv) * per_head + (pos >> chunk_shift) + row;
}
// A row [rb, re) of a caller's CSR is used only if 0 <= rb <= re <= cap. Each used row
// then reads and slots inside the tables, and when every row of a KV head passes, its
// row starts are non-decreasing within [0, cap], so kv_item_slot's slots are distinct
// and each key's count is exact; a failing row voids the whole item order (sb.bad).
__host__ __device__ inline bool kv_row_ok(long long rb, long long re, long long cap) {
  return rb >= 0 && rb <= re && re <= cap;
}
// Key of a kv-centric work item: its KV head and first query as one coordinate
// c = hkv * nq + first query, bucketed into kKvKeys equal ranges; stream s of the
// kernel holds keys [s * kKvKeys / streams, (s + 1) * kKvKeys / streams).
__device__ __forceinline__ int kv_item_key(int hkv, long long first_q, long long nq, int Hkv) {
  return query_bucket(static_cast<long long>(hkv) * nq + first_q, static_cast<long long>(Hkv) * nq,
                      kKvKeys);
}
// items for every chunk of 2^chunk_shift entries of every CSR row of a caller's CSR,
// each at its slot (kv_item_slot), and the per-key item counts (q_idx [Hkv][cap]
// holding query * qdiv + slot, qdiv = 1 for plain query ids; nq query rows; the
// table and the sort buffers' zero region cleared beforehand)
hipError_t launch_kv_items(const int32_t* row_ptr, int Hkv, int nrows, int chunk_shift,
                           long long per_head, int4* items, const int32_t* q_idx, long long cap,
                           long long nq, int qdiv, const KvSortBuffers& sb, hipStream_t stream);
// the item table (max_items slots, unused ones with entry count 0) in key order; the
// item count and key_start are computed on the device from sb.counts
hipError_t launch_kv_items_by_key(const int4* items, int Hkv, const int32_t* q_idx, long long cap,
                                  long long nq, int qdiv, long long max_items,
                                  const KvSortBuffers& sb, int4* out, hipStream_t stream);
// zero n0 ints at p0 and n1 at p1 (a fill kernel, so that a captured graph holds no
// memset node)
hipError_t launch_zero_ints(int32_t* p0, long long n0, int32_t* p1, long long n1,
                            hipStream_t stream);
// compute units of the current device (cached per device)
int device_cu_count();

// combine of slot partials (kv-centric): valid slots are the q2k entries in [0, nblk)
// (uniform batch), or in [0, ceil(Skv_b / 128)) for a varlen batch (v != nullptr)
struct CombineVarlen {
  const int2* q_rows;  // VarlenTables::q_rows
};
// lse_t_part / lse_t (both or neither): merge of the temperature-scaled block LSEs
hipError_t launch_combine_slots(const uint16_t* o_part, const float2* lse_part, const int32_t* q2k,
                                int B, int Sq, int Hq, int Hkv, int topk, int nblk, uint16_t* o,
                                float* lse, hipStream_t stream, const CombineVarlen* v = nullptr,
                                const float* lse_t_part = nullptr, float* lse_t = nullptr);
// combine of split partials (split-KV q-centric / paged decode)
hipError_t launch_combine_splits(const float* o_part, const float* lse_part, int B, int Sq, int Hq,
                                 int splits, uint16_t* o, float* lse, hipStream_t stream,
                                 const float* lse_t_part = nullptr, float* lse_t = nullptr);

// exclusive scan of n int32 values: out[0..n] (out[n] = total); tmp >= scan_tmp_ints(n) ints
size_t scan_tmp_ints(long long n);
hipError_t launch_exclusive_scan(const int32_t* in, int32_t* out, long long n, int32_t* tmp,
                                 hipStream_t stream);

struct CsrPlan {
  int ntiles;        // query tiles per KV head
  int tile_q;        // queries per tile
  long long counts;  // Hkv * nrows * ntiles
};
CsrPlan csr_plan(int B, int Hkv, int Sq, int topk, int nrows);
size_t csr_workspace_bytes(int B, int Hkv, int Sq, int topk, int nrows);
// ordered = true: entries of a row ascending in (query, slot), the unique CSR
// ordered = false: same rows and entry sets, order inside a row unspecified
// (used internally by the kv-centric path, whose results do not depend on it)
// flat (ordered = false only, B*Sq*topk < 2^31): q_idx holds each entry as its index
// query * topk + slot into the KV head's index table; slot is not written
// The kv-centric work items, listed by the order-free flat build while it scatters:
// the entry that lands first in a chunk of 2^chunk_shift entries of its row writes the
// chunk's item (hkv, row, position, entry count) to its slot (kv_item_slot) and counts
// it under its key (kv_item_key of the entry's query) in sb.counts. The count pass
// clears the table (max_items int4) and the sort buffers' zero region first.
struct KvItemEmit {
  int4* items;
  long long per_head;
  long long max_items;
  KvSortBuffers sb;
  int chunk_shift;
};
hipError_t launch_build_csr(const int32_t* q2k, int B, int Hkv, int Sq, int topk, int nblk,
                            int32_t* row_ptr, int32_t* q_idx, int32_t* slot, void* ws,
                            hipStream_t stream, bool ordered = true, bool flat = false,
                            const KvItemEmit* emit = nullptr);
// varlen CSR over nrows rows (q2k [Hkv,total_q,topk]); the tables come from
// launch_varlen_tables; entries whose row is >= nrows are dropped. Workspace:
// csr_workspace_bytes(1, Hkv, total_q, topk, nrows).
hipError_t launch_build_csr_varlen(const int32_t* q2k, const VarlenTables& t, int Hkv,
                                   int total_q, int topk,
                                   int nrows, int32_t* row_ptr, int32_t* q_idx, int32_t* slot,
                                   void* ws, hipStream_t stream, bool ordered = true,
                                   bool flat = false, const KvItemEmit* emit = nullptr);

}  // namespace msa
