// kv-block -> query CSR builder and device exclusive scan; the order-free build
// also lists the kv-centric work items (one per chunk of each row) as it scatters.
//
// The CSR is the one `build_k2q_csr` produces on the page "MSA interface.py"
// (row r = b * nblk + s of each KV head lists the global query ids b*Sq + q
// whose index row selects block s; the page "test_sparse_atten.py" checks it
// bit-exact against a reference). Entries are ordered by query, then slot, so
// the result is unique and every call writes the same bits.
//
// A variable-length batch (q2k [Hkv, total_q, topk], `build_k2q_csr` with
// cu_seqlens and total_rows) has the same passes: query g of sequence b maps
// slot value s in [0, ceil(Skv_b / 128)) to row rowbase[b] + s, read from the
// per-query table of (rowbase[b], block count).
//
// Method (a stable counting sort, no order-dependent atomics):
//   1. count:   the entry sequence of each KV head, in (query, slot) order, is
//               cut into tiles of whole queries; each tile histograms its rows
//               in LDS (commutative adds) into counts[hkv][row][tile].
//   2. scan:    one exclusive scan of counts in (hkv, row, tile) order gives
//               every (row, tile) its first output position.
//   3. scatter: one wave per tile walks its entries in order, 64 at a time;
//               entries of one batch that share a row are ranked by ballot /
//               popcount (lower lane first), and a per-row cursor in LDS
//               carries the offset from batch to batch.
//   4. row_ptr: read off the scanned counts at tile 0 of each row.
#include "msa_internal.hpp"

#include <algorithm>

namespace msa {

namespace {

constexpr int kScanThreads = 256;
constexpr int kScanItems = 8;
constexpr int kScanTile = kScanThreads * kScanItems;

// exclusive scan of one value per thread across a 256-thread block; returns the
// block total in *total
__device__ int block_exclusive_scan(int v, int* total) {
  __shared__ int wave_sums[kScanThreads / 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wave_sums[wave] = x;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kScanThreads / 64; ++w) {
    if (w < wave) before += wave_sums[w];
    all += wave_sums[w];
  }
  __syncthreads();
  *total = all;
  return before + x - v;
}

__global__ __launch_bounds__(kScanThreads) void scan_tile_sums(const int32_t* in, long long n,
                                                               int32_t* sums) {
  const long long base = static_cast<long long>(blockIdx.x) * kScanTile;
  int acc = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const long long k = base + static_cast<long long>(threadIdx.x) * kScanItems + i;
    if (k < n) acc += in[k];
  }
  int total;
  block_exclusive_scan(acc, &total);
  if (threadIdx.x == 0) sums[blockIdx.x] = total;
}

// single block: exclusive scan of the tile sums, in place
__global__ __launch_bounds__(kScanThreads) void scan_tile_offsets(int32_t* sums, int ntiles) {
  int carry = 0;
  for (int base = 0; base < ntiles; base += kScanTile) {
    int v[kScanItems];
    int acc = 0;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int k = base + threadIdx.x * kScanItems + i;
      v[i] = k < ntiles ? sums[k] : 0;
      acc += v[i];
    }
    int total;
    int run = block_exclusive_scan(acc, &total) + carry;
#pragma unroll
    for (int i = 0; i < kScanItems; ++i) {
      const int k = base + threadIdx.x * kScanItems + i;
      if (k < ntiles) sums[k] = run;
      run += v[i];
    }
    carry += total;
    __syncthreads();
  }
}

__global__ __launch_bounds__(kScanThreads) void scan_apply(const int32_t* in, long long n,
                                                           const int32_t* offsets, int32_t* out) {
  const long long base = static_cast<long long>(blockIdx.x) * kScanTile;
  int v[kScanItems];
  int acc = 0;
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const long long k = base + static_cast<long long>(threadIdx.x) * kScanItems + i;
    v[i] = k < n ? in[k] : 0;
    acc += v[i];
  }
  int total;
  int run = block_exclusive_scan(acc, &total) + offsets[blockIdx.x];
#pragma unroll
  for (int i = 0; i < kScanItems; ++i) {
    const long long k = base + static_cast<long long>(threadIdx.x) * kScanItems + i;
    if (k < n) out[k] = run;
    run += v[i];
  }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == kScanThreads - 1) out[n] = run;
}

// ---------------------------------------------------------------------------
// CSR passes. Grid (ntiles, Hkv). Tile `tile` of KV head hkv covers global
// queries [tile * tile_q, min(nq, (tile+1) * tile_q)).
// ---------------------------------------------------------------------------
struct CsrSrc {
  const int32_t* q2k;
  const int2* q_rows;  // varlen: (first row, block count) of each query's sequence
  int Hkv, Sq, topk, nblk, nrows;
  long long nq;        // B * Sq, or total_q
};

// n / d for an entry or query index. With I32 (every entry index of the build below
// 2^31) it is the 32-bit unsigned division, a short instruction sequence; the 64-bit
// one is a long software routine and dominated the count and scatter kernels.
template <bool I32>
__device__ __forceinline__ long long idx_div(long long n, int d) {
  if constexpr (I32)
    return static_cast<long long>(static_cast<uint32_t>(n) / static_cast<uint32_t>(d));
  else
    return n / d;
}

// CSR row of entry e = (query, slot) of KV head hkv, or -1 when its slot is unused
template <bool VARLEN, bool I32>
__device__ __forceinline__ int entry_row(const CsrSrc& a, int hkv, long long e) {
  const long long gq = idx_div<I32>(e, a.topk);
  if (VARLEN) {
    const int s = a.q2k[static_cast<long long>(hkv) * a.nq * a.topk + e];
    const int2 qr = a.q_rows[gq];
    if (s < 0 || s >= qr.y) return -1;
    const long long r = static_cast<long long>(qr.x) + s;
    return r < a.nrows ? static_cast<int>(r) : -1;
  } else {
    const int t = static_cast<int>(e - gq * a.topk);
    const int b = static_cast<int>(idx_div<I32>(gq, a.Sq));
    const int qpos = static_cast<int>(gq - static_cast<long long>(b) * a.Sq);
    const int s = a.q2k[((static_cast<long long>(b) * a.Hkv + hkv) * a.Sq + qpos) * a.topk + t];
    return (s >= 0 && s < a.nblk) ? b * a.nblk + s : -1;
  }
}

// Stable rank of each lane among the lower lanes holding the same row, and the
// number of lanes holding it (row < 0: not counted). One pass per distinct row:
// the lowest pending lane's row is read with v_readlane (no LDS round trip) and its
// peers found by one ballot.
__device__ __forceinline__ void rank_in_batch(int row, int& rank, int& cnt) {
  unsigned long long pending = __ballot(row >= 0);
  const unsigned long long below = __lanemask_lt();
  while (pending) {
    const int leader = __ffsll(static_cast<long long>(pending)) - 1;
    const int lrow = __builtin_amdgcn_readlane(row, leader);
    const unsigned long long peers = __ballot(row == lrow);
    const bool mine = row == lrow;
    rank = mine ? __popcll(peers & below) : rank;
    cnt = mine ? __popcll(peers) : cnt;
    pending &= ~peers;
  }
}

constexpr int kCsrBatch = 8;  // entries per thread whose index loads are in flight together
constexpr size_t kCsrMaskLdsMax = 150 * 1024;  // LDS of the mask-ranked scatter, at most

// How the ordered scatter ranks a wave's 64-entry batch: by ballots per distinct row; with
// a per-row table of lane masks in LDS; or with a small per-wave hash table of (row, mask)
// slots, which needs no per-row table, so that wide tables leave room for more
// workgroups per compute unit.
enum CsrRank { kRankBallot = 0, kRankMask = 1, kRankHash = 2 };
constexpr int kCsrHashSlots = 128;  // per wave; a batch holds at most 64 distinct rows
// Tables of more rows than this rank by hash. Public build, ms, mask / hash ranking (the
// same bits): 64 rows 0.024 / 0.026, 256 rows 0.045 / 0.047, 384 rows 0.035 / 0.037,
// 3072 rows 0.219 / 0.189 (one workgroup per compute unit with the masks, two with the
// slots), 8000 rows 0.250 / 0.059 (past the mask tables' LDS the one-wave scatter ran).
constexpr int kCsrHashAboveRows = 2048;

// Query tile of workgroup x. Workgroups are dealt round-robin over the 8 XCDs, and
// consecutive tiles write adjacent counts and adjacent runs of a row's entries, so
// the tiles are permuted to run in groups of ntiles / 8 consecutive tiles per XCD:
// a cache line that several tiles fill is then merged in one XCD's L2 instead of
// being written back in pieces from several. The last ntiles % 8 keep their place.
__device__ __forceinline__ int csr_tile_of(int x, int ntiles) {
  const int per = ntiles >> 3;
  return x < 8 * per ? (x & 7) * per + (x >> 3) : x;
}

// rows[k] = CSR row of entry e0 + stride k, or -1 from e_end on (e0 < e_end). The
// index is clamped into range so that every load is unconditional and all N are in
// flight together: a load under a branch is waited for where the branch joins.
template <bool VARLEN, bool I32, int N>
__device__ __forceinline__ void load_rows(const CsrSrc& a, int hkv, long long e0, int stride,
                                          long long e_end, int (&rows)[N]) {
#pragma unroll
  for (int k = 0; k < N; ++k) {
    const long long e = e0 + static_cast<long long>(stride) * k;
    const int r = entry_row<VARLEN, I32>(a, hkv, e < e_end ? e : e_end - 1);
    rows[k] = e < e_end ? r : -1;
  }
}

// Fill of zeros over two int ranges, shared out over all workgroups of the grid.
__device__ __forceinline__ void grid_zero2(int32_t* p0, long long n0, int32_t* p1, long long n1) {
  const long long nb = static_cast<long long>(gridDim.x) * gridDim.y;
  const long long b = static_cast<long long>(blockIdx.y) * gridDim.x + blockIdx.x;
  for (long long i = b * blockDim.x + threadIdx.x; i < n0 + n1; i += nb * blockDim.x) {
    if (i < n0) p0[i] = 0;
    else p1[i - n0] = 0;
  }
}

// z: ranges the grid also clears (the kv-centric item table and its counters, filled
// by the scatter that follows)
struct ZeroRanges {
  int32_t* p0;
  long long n0;
  int32_t* p1;
  long long n1;
};

template <bool VARLEN, bool I32, int NT>
__global__ __launch_bounds__(NT) void csr_count_kernel(CsrSrc a, int tile_q, int ntiles,
                                                        int32_t* __restrict__ counts,
                                                        ZeroRanges z) {
  extern __shared__ int cnt[];
  const int tile = csr_tile_of(blockIdx.x, ntiles), hkv = blockIdx.y;
  const int nrows = a.nrows;
  if (z.n0 + z.n1 > 0) grid_zero2(z.p0, z.n0, z.p1, z.n1);
  for (int r = threadIdx.x; r < nrows; r += blockDim.x) cnt[r] = 0;
  __syncthreads();
  const long long g0 = static_cast<long long>(tile) * tile_q;
  const long long g1 = std::min<long long>(a.nq, g0 + tile_q);
  const long long e1 = g1 * a.topk;
  // kCsrBatch entries per thread per round, their index loads issued together
  for (long long rb = g0 * a.topk; rb < e1; rb += NT * kCsrBatch) {
    int rows[kCsrBatch];
    load_rows<VARLEN, I32>(a, hkv, rb + threadIdx.x, NT, e1, rows);
#pragma unroll
    for (int k = 0; k < kCsrBatch; ++k)
      if (rows[k] >= 0) atomicAdd(&cnt[rows[k]], 1);
  }
  __syncthreads();
  for (int r = threadIdx.x; r < nrows; r += blockDim.x)
    counts[(static_cast<long long>(hkv) * nrows + r) * ntiles + tile] = cnt[r];
}

// Stable scatter, one wave per (tile, KV head): the tile's entries are taken in
// rounds of 64 x 16 (all loads of a round issued together), then in order in
// batches of 64 consecutive entries; a lane's rank among the lower lanes holding
// the same row comes from ballots (one pass per distinct row in the batch), so
// entries of a row keep ascending (query, slot) order.
template <bool VARLEN, bool I32>
__global__ __launch_bounds__(64) void csr_scatter_kernel(CsrSrc a, int tile_q, int ntiles,
                                                         const int32_t* __restrict__ offsets,
                                                         int32_t* __restrict__ q_idx,
                                                         int32_t* __restrict__ slot) {
  extern __shared__ int cursor[];
  constexpr int kPer = 16;  // entries per lane per round
  const int tile = csr_tile_of(blockIdx.x, ntiles), hkv = blockIdx.y;
  const int lane = threadIdx.x;
  const int nrows = a.nrows;
  const long long cap = a.nq * a.topk;
  const long long seg = static_cast<long long>(hkv) * nrows * ntiles;
  const int base_h = offsets[seg];
  for (int r = lane; r < nrows; r += 64)
    cursor[r] = offsets[seg + static_cast<long long>(r) * ntiles + tile] - base_h;
  __syncthreads();
  const long long g0 = static_cast<long long>(tile) * tile_q;
  const long long g1 = std::min<long long>(a.nq, g0 + tile_q);
  const long long e_end = g1 * a.topk;
  int32_t* qi = q_idx + hkv * cap;
  int32_t* sl = slot ? slot + hkv * cap : nullptr;
  for (long long rb = g0 * a.topk; rb < e_end; rb += 64 * kPer) {
    int rows[kPer];
    load_rows<VARLEN, I32>(a, hkv, rb + lane, 64, e_end, rows);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const long long e = rb + 64 * k + lane;
      const int row = rows[k];
      int rank = 0, cnt = 0;
      rank_in_batch(row, rank, cnt);
      int pos = 0;
      if (row >= 0) pos = cursor[row] + rank;
      __syncthreads();
      if (row >= 0 && rank == cnt - 1) cursor[row] = pos + 1;
      if (row >= 0) {
        const long long q = idx_div<I32>(e, a.topk);
        qi[pos] = static_cast<int32_t>(q);
        if (sl) sl[pos] = static_cast<int32_t>(e - q * a.topk);
      }
      __syncthreads();
    }
  }
}

// The same stable scatter with four waves per (tile, KV head): wave w takes the
// w-th quarter of the tile's queries. The waves first histogram their quarters
// into their own LDS counters; an exclusive prefix over the waves then gives each
// wave, per row, the position after the entries of the lower quarters; each wave
// finally runs the ballot-ranked scatter above on its quarter. Same output bits,
// four times the waves. LDS: 4 * nrows ints.
//
// kRankMask: the lanes of a batch find the peers holding their row through a
// per-wave table of 64-bit lane masks in LDS (each lane ORs its bit into its row's
// mask and reads it back; the row's last lane clears it), in a constant number of
// steps instead of one ballot pass per distinct row of the batch: on wide tables
// nearly every entry of a batch has a row of its own. LDS: 4 * nrows * (4 + 8) bytes.
// kRankHash: the same masks kept in kCsrHashSlots (row, mask) slots per wave instead
// of one per row. LDS: 4 * nrows * 4 + 4 * kCsrHashSlots * (8 + 4) bytes.
template <bool VARLEN, bool I32, int RANK>
__global__ __launch_bounds__(256) void csr_scatter4_kernel(CsrSrc a, int tile_q, int ntiles,
                                                           const int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ q_idx,
                                                           int32_t* __restrict__ slot) {
  extern __shared__ __attribute__((aligned(8))) int lds[];
  constexpr int kPer = 16;  // entries per lane per round
  const int tile = csr_tile_of(blockIdx.x, ntiles), hkv = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nrows = a.nrows;
  const long long cap = a.nq * a.topk;
  const long long seg = static_cast<long long>(hkv) * nrows * ntiles;
  const long long g0 = static_cast<long long>(tile) * tile_q;
  const long long g1 = std::min<long long>(a.nq, g0 + tile_q);
  const long long sub = (g1 - g0 + 3) / 4;
  const long long w0 = std::min(g1, g0 + wave * sub), w1 = std::min(g1, w0 + sub);
  int* cursor = lds + wave * nrows;
  // kRankMask: the waves' mask tables follow the 4 * nrows cursors (8-byte aligned:
  // nrows is rounded up to even); kRankHash: there the waves' hash slots instead, each
  // a row (-1 = empty) and a lane mask
  unsigned long long* tables = reinterpret_cast<unsigned long long*>(lds + 4 * ((nrows + 1) & ~1));
  unsigned long long* mask = tables + wave * nrows;
  unsigned long long* hmask = tables + wave * kCsrHashSlots;
  int* hkey = reinterpret_cast<int*>(tables + 4 * kCsrHashSlots) + wave * kCsrHashSlots;
  for (int r = tid; r < 4 * nrows; r += 256) lds[r] = 0;
  if (RANK == kRankMask)
    for (int r = tid; r < 4 * nrows; r += 256) tables[r] = 0;
  if (RANK == kRankHash)
    for (int r = tid; r < 4 * kCsrHashSlots; r += 256) {
      tables[r] = 0;
      reinterpret_cast<int*>(tables + 4 * kCsrHashSlots)[r] = -1;
    }
  __syncthreads();
  for (long long rb = w0 * a.topk; rb < w1 * a.topk; rb += 64 * kCsrBatch) {
    int rows[kCsrBatch];
    load_rows<VARLEN, I32>(a, hkv, rb + lane, 64, w1 * a.topk, rows);
#pragma unroll
    for (int k = 0; k < kCsrBatch; ++k)
      if (rows[k] >= 0) atomicAdd(&cursor[rows[k]], 1);
  }
  __syncthreads();
  const int base_h = offsets[seg];
  for (int r = tid; r < nrows; r += 256) {
    int run = offsets[seg + static_cast<long long>(r) * ntiles + tile] - base_h;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int c = lds[w * nrows + r];
      lds[w * nrows + r] = run;
      run += c;
    }
  }
  __syncthreads();
  const long long e_end = w1 * a.topk;
  int32_t* qi = q_idx + hkv * cap;
  int32_t* sl = slot ? slot + hkv * cap : nullptr;
  for (long long rb = w0 * a.topk; rb < e_end; rb += 64 * kPer) {
    int rows[kPer];
    load_rows<VARLEN, I32>(a, hkv, rb + lane, 64, e_end, rows);
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const long long e = rb + 64 * k + lane;
      const int row = rows[k];
      int rank = 0, cnt = 0, hs = 0;
      if (RANK == kRankMask) {
        // one wave, LDS accesses in program order: every OR lands before the reads
        if (row >= 0) atomicOr(&mask[row], 1ull << lane);
        __builtin_amdgcn_wave_barrier();
        if (row >= 0) {
          const unsigned long long peers = mask[row];
          rank = __popcll(peers & __lanemask_lt());
          cnt = __popcll(peers);
        }
      } else if (RANK == kRankHash) {
        // claim the row's slot (linear probing from a multiplicative hash; the table
        // never holds more than 64 rows, so every lane finds its row or an empty slot
        // within kCsrHashSlots probes), then OR the lane into the slot's mask
        if (row >= 0) {
          hs = static_cast<int>((static_cast<uint32_t>(row) * 2654435761u) >> 25);
          for (int probe = 0; probe < kCsrHashSlots; ++probe) {
            const int prev = atomicCAS(&hkey[hs], -1, row);
            if (prev == -1 || prev == row) break;
            hs = (hs + 1) & (kCsrHashSlots - 1);
          }
          atomicOr(&hmask[hs], 1ull << lane);
        }
        __builtin_amdgcn_wave_barrier();
        if (row >= 0) {
          const unsigned long long peers = hmask[hs];
          rank = __popcll(peers & __lanemask_lt());
          cnt = __popcll(peers);
        }
      } else {
        rank_in_batch(row, rank, cnt);
      }
      // this wave's cursors only: its lanes read before the last-ranked lane of a row
      // writes (one wave, LDS accesses in program order)
      int pos = 0;
      if (row >= 0) pos = cursor[row] + rank;
      __builtin_amdgcn_wave_barrier();
      if (row >= 0 && rank == cnt - 1) {
        cursor[row] = pos + 1;
        if (RANK == kRankMask) mask[row] = 0;
        if (RANK == kRankHash) {  // every lane of the row has read the mask: free the slot
          hmask[hs] = 0;
          hkey[hs] = -1;
        }
      }
      if (row >= 0) {
        const long long q = idx_div<I32>(e, a.topk);
        qi[pos] = static_cast<int32_t>(q);
        if (sl) sl[pos] = static_cast<int32_t>(e - q * a.topk);
      }
      __builtin_amdgcn_wave_barrier();
    }
  }
}

// Unordered scatter: every entry of a (row, tile) segment lands inside that
// segment, slot claimed with an LDS atomic (order within a segment unspecified).
// LDS: nrows cursors (at most kMaxCsrRows ints), and with ITEMS each row's first
// position and a histogram of the listed items' keys beside them.
// FLAT: each entry is stored as its index e = query * topk + slot into the KV head's
// index table (one int32 instead of a query and a slot); slot is unused.
// ITEMS: the entry that lands on the first position of a chunk of 2^chunk_shift
// entries of its row writes the chunk's kv-centric work item to its slot (KvItemEmit);
// the workgroup's item counts per key go out at its end, one atomic per key used.
template <bool VARLEN, bool I32, bool FLAT, bool ITEMS>
__global__ __launch_bounds__(256) void csr_scatter_unordered_kernel(
    CsrSrc a, int tile_q, int ntiles, const int32_t* __restrict__ offsets,
    int32_t* __restrict__ q_idx, int32_t* __restrict__ slot, int32_t* __restrict__ row_ptr,
    KvItemEmit emit) {
  extern __shared__ int cursor[];
  const int tile = csr_tile_of(blockIdx.x, ntiles), hkv = blockIdx.y;
  const int nrows = a.nrows;
  int* rowbeg = cursor + nrows;  // ITEMS only
  int* hist = rowbeg + nrows;    // ITEMS only: [kKvKeys]
  const long long cap = a.nq * a.topk;
  const long long seg = static_cast<long long>(hkv) * nrows * ntiles;
  const int base_h = offsets[seg];
  for (int r = threadIdx.x; r < nrows; r += blockDim.x) {
    cursor[r] = offsets[seg + static_cast<long long>(r) * ntiles + tile] - base_h;
    if (ITEMS) rowbeg[r] = offsets[seg + static_cast<long long>(r) * ntiles] - base_h;
    // tile 0 holds each row's first position: the row pointers of this KV head
    if (row_ptr && tile == 0) row_ptr[static_cast<long long>(hkv) * (nrows + 1) + r] = cursor[r];
  }
  if (ITEMS)
    for (int i = threadIdx.x; i < kKvKeys; i += blockDim.x) hist[i] = 0;
  if (row_ptr && tile == 0 && threadIdx.x == 0)
    row_ptr[static_cast<long long>(hkv) * (nrows + 1) + nrows] =
        offsets[seg + static_cast<long long>(nrows) * ntiles] - base_h;
  __syncthreads();
  const long long g0 = static_cast<long long>(tile) * tile_q;
  const long long g1 = std::min<long long>(a.nq, g0 + tile_q);
  int32_t* qi = q_idx + hkv * cap;
  int32_t* sl = slot ? slot + hkv * cap : nullptr;
  const long long e1 = g1 * a.topk;
  const int cmask = ITEMS ? (1 << emit.chunk_shift) - 1 : 0;
  for (long long rb = g0 * a.topk; rb < e1; rb += 256 * kCsrBatch) {
    int rows[kCsrBatch], pos[kCsrBatch];
    load_rows<VARLEN, I32>(a, hkv, rb + threadIdx.x, 256, e1, rows);
    // every atomic is issued before any result is used; an unused slot adds 0 to
    // row 0's cursor, which leaves it unchanged
#pragma unroll
    for (int k = 0; k < kCsrBatch; ++k)
      pos[k] = atomicAdd(&cursor[rows[k] >= 0 ? rows[k] : 0], rows[k] >= 0 ? 1 : 0);
#pragma unroll
    for (int k = 0; k < kCsrBatch; ++k) {
      if (rows[k] < 0) continue;
      const long long e = rb + 256 * k + threadIdx.x;
      if (ITEMS && ((pos[k] - rowbeg[rows[k]]) & cmask) == 0) {
        // first entry of a chunk: the chunk's work item (the row ends where the next
        // row's tile 0 begins)
        const int end =
            offsets[seg + static_cast<long long>(rows[k] + 1) * ntiles] - base_h;
        emit.items[kv_item_slot(hkv, emit.per_head, pos[k], emit.chunk_shift, rows[k])] =
            make_int4(hkv, rows[k], pos[k], min(cmask + 1, end - pos[k]));
        atomicAdd(&hist[kv_item_key(hkv, idx_div<I32>(e, a.topk), a.nq, a.Hkv)], 1);
      }
      if (FLAT) {
        qi[pos[k]] = static_cast<int32_t>(e);
        continue;
      }
      const long long q = idx_div<I32>(e, a.topk);
      qi[pos[k]] = static_cast<int32_t>(q);
      if (sl) sl[pos[k]] = static_cast<int32_t>(e - q * a.topk);
    }
  }
  if (ITEMS) {
    __syncthreads();
    for (int i = threadIdx.x; i < kKvKeys; i += blockDim.x) {
      const int n = hist[i];
      if (n) atomicAdd(&emit.sb.counts[i], n);
    }
  }
}

__global__ void csr_row_ptr_kernel(const int32_t* __restrict__ offsets, int Hkv, int nrows,
                                   int ntiles, int32_t* __restrict__ row_ptr) {
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx >= static_cast<long long>(Hkv) * (nrows + 1)) return;
  const int hkv = static_cast<int>(idx / (nrows + 1)), r = static_cast<int>(idx % (nrows + 1));
  const long long seg = static_cast<long long>(hkv) * nrows * ntiles;
  row_ptr[idx] = offsets[seg + static_cast<long long>(r) * ntiles] - offsets[seg];
}

inline unsigned blocks_for(long long n, int per) { return static_cast<unsigned>((n + per - 1) / per); }

__global__ void zero_ints_kernel(int32_t* __restrict__ p0, long long n0, int32_t* __restrict__ p1,
                                 long long n1) {
  grid_zero2(p0, n0, p1, n1);
}

// Exclusive scan of at most kScanOneMax values in one workgroup of 1024 threads. Tile j
// holds values [4096 j, 4096 (j + 1)); thread t loads and stores its four values of
// each tile as one 16-byte vector (coalesced across the wave). Each wave scans its
// 256 values of a tile with lane shuffles; one wave then scans the (tile, wave)
// totals in order, which gives every wave's run its offset. out[n] = the total.
constexpr int kScanOneThreads = 1024;
constexpr int kScanOneTiles = 16;
constexpr long long kScanOneMax = 4LL * kScanOneThreads * kScanOneTiles;
__global__ __launch_bounds__(kScanOneThreads) void scan_one_block_kernel(
    const int32_t* __restrict__ in, int n, int32_t* __restrict__ out) {
  constexpr int kWaves = kScanOneThreads / 64;
  __shared__ int blk[kScanOneTiles * kWaves];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int T = (n + 4 * kScanOneThreads - 1) / (4 * kScanOneThreads);
  int4 v[kScanOneTiles];
  int pre[kScanOneTiles];
#pragma unroll
  for (int j = 0; j < kScanOneTiles; ++j) {
    v[j] = make_int4(0, 0, 0, 0);
    pre[j] = 0;
    if (j < T) {
      const int k = j * 4 * kScanOneThreads + 4 * t;
      if (k + 3 < n) {
        v[j] = *reinterpret_cast<const int4*>(in + k);
      } else {
        v[j].x = k < n ? in[k] : 0;
        v[j].y = k + 1 < n ? in[k + 1] : 0;
        v[j].z = k + 2 < n ? in[k + 2] : 0;
      }
      const int own = v[j].x + v[j].y + v[j].z + v[j].w;
      int x = own;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(x, d);
        if (lane >= d) x += y;
      }
      pre[j] = x - own;
      if (lane == 63) blk[j * kWaves + wave] = x;
    }
  }
  __syncthreads();
  if (wave == 0) {  // exclusive scan of the T * kWaves (tile, wave) totals, 4 per lane
    int a[4], own = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = 4 * lane + i < T * kWaves ? blk[4 * lane + i] : 0;
      own += a[i];
    }
    int x = own;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    int run = x - own;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (4 * lane + i < T * kWaves) blk[4 * lane + i] = run;
      run += a[i];
    }
    if (lane == 63) out[n] = x;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kScanOneTiles; ++j) {
    if (j < T) {
      const int k = j * 4 * kScanOneThreads + 4 * t;
      const int b = blk[j * kWaves + wave] + pre[j];
      const int4 o = make_int4(b, b + v[j].x, b + v[j].x + v[j].y, b + v[j].x + v[j].y + v[j].z);
      if (k + 3 < n) {
        *reinterpret_cast<int4*>(out + k) = o;
      } else {
        if (k < n) out[k] = o.x;
        if (k + 1 < n) out[k + 1] = o.y;
        if (k + 2 < n) out[k + 2] = o.z;
      }
    }
  }
}

}  // namespace

size_t scan_tmp_ints(long long n) { return static_cast<size_t>((n + kScanTile - 1) / kScanTile) + 1; }

hipError_t launch_exclusive_scan(const int32_t* in, int32_t* out, long long n, int32_t* tmp,
                                 hipStream_t stream) {
  if (n <= 0) return hipErrorInvalidValue;
  if (n <= kScanOneMax && (reinterpret_cast<uintptr_t>(in) | reinterpret_cast<uintptr_t>(out)) % 16 == 0) {
    hipLaunchKernelGGL(scan_one_block_kernel, dim3(1), dim3(kScanOneThreads), 0, stream, in,
                       static_cast<int>(n), out);
    return hipGetLastError();
  }
  const long long ntiles = (n + kScanTile - 1) / kScanTile;
  if (ntiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(scan_tile_sums, dim3(static_cast<unsigned>(ntiles)), dim3(kScanThreads), 0,
                     stream, in, n, tmp);
  hipLaunchKernelGGL(scan_tile_offsets, dim3(1), dim3(kScanThreads), 0, stream, tmp,
                     static_cast<int>(ntiles));
  hipLaunchKernelGGL(scan_apply, dim3(static_cast<unsigned>(ntiles)), dim3(kScanThreads), 0,
                     stream, in, n, tmp, out);
  return hipGetLastError();
}

// Query tiles of the CSR passes: about tile_queries queries each, and never more than
// 4M (KV head, row, tile) counts.
static CsrPlan csr_plan_tiles(long long nq, int Hkv, int nrows, int tile_queries) {
  long long ntiles = (nq + tile_queries - 1) / tile_queries;
  const long long max_counts = 4LL << 20;
  const long long cap_tiles = std::max<long long>(1, max_counts / (static_cast<long long>(Hkv) * nrows));
  ntiles = std::max<long long>(1, std::min(ntiles, cap_tiles));
  CsrPlan plan;
  plan.tile_q = static_cast<int>((nq + ntiles - 1) / ntiles);
  plan.ntiles = static_cast<int>((nq + plan.tile_q - 1) / plan.tile_q);
  plan.counts = static_cast<long long>(Hkv) * nrows * plan.ntiles;
  return plan;
}

// The published plan (it sizes the workspace): ~64 queries per tile, the most tiles any
// build uses.
CsrPlan csr_plan(int B, int Hkv, int Sq, int topk, int nrows) {
  (void)topk;
  return csr_plan_tiles(static_cast<long long>(B) * Sq, Hkv, nrows, 64);
}

// Queries per tile of the ordered (public) build: longer tiles give each workgroup of the
// ranked scatter more entries for its fixed cost of clearing and reading its tables.
// Public build, ms, at 64 / 256 / 1024 queries per tile (the same bits at every size):
// 8192 causal queries, 4 KV heads, topk 16: 0.026 / 0.024 / 0.050; 32768 queries, 4 KV
// heads, topk 16: 0.056 / 0.045 / 0.063; 49152 causal queries, 1 KV head: 0.033 / 0.033 /
// 0.054. Tables of 3072 rows keep the tile count of the 4M-count cap either way.
constexpr int kCsrOrderedTileQ = 256;

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

size_t csr_workspace_bytes(int B, int Hkv, int Sq, int topk, int nrows) {
  const CsrPlan plan = csr_plan(B, Hkv, Sq, topk, nrows);
  return align256(plan.counts * 4) + align256((plan.counts + 1) * 4) +
         align256(scan_tmp_ints(plan.counts) * 4);
}

namespace {

// Tiles of the order-free build: long enough that a (row, tile) segment averages
// at least 8 entries, a 32-byte run of q_idx and of slot, so that the scatter's
// 4-byte stores fill whole sectors instead of each landing in a line of its own
// (with 3072 rows and ~64-query tiles a segment holds one or two entries). Never
// more tiles, hence never more counts, than the published plan, which sizes the
// workspace.
CsrPlan csr_plan_unordered(int Hkv, long long nq, int topk, int nrows) {
  CsrPlan plan = csr_plan(1, Hkv, static_cast<int>(nq), topk, nrows);
  const long long want = std::min<long long>(nq, (8LL * nrows + topk - 1) / topk);
  if (want > plan.tile_q) {
    plan.tile_q = static_cast<int>(want);
    plan.ntiles = static_cast<int>((nq + want - 1) / want);
    plan.counts = static_cast<long long>(Hkv) * nrows * plan.ntiles;
  }
  return plan;
}

template <bool VARLEN, bool I32>
hipError_t build_csr_impl(const CsrSrc& a, int32_t* row_ptr, int32_t* q_idx, int32_t* slot,
                          void* ws, hipStream_t stream, bool ordered, bool flat,
                          const KvItemEmit* emit) {
  const int nrows = a.nrows;
  // the plan depends on the query count and the rows only: B * Sq == nq
  const CsrPlan plan = ordered ? csr_plan_tiles(a.nq, a.Hkv, nrows, kCsrOrderedTileQ)
                               : csr_plan_unordered(a.Hkv, a.nq, a.topk, nrows);
  char* base = static_cast<char*>(ws);
  int32_t* counts = reinterpret_cast<int32_t*>(base);
  base += align256(plan.counts * 4);
  int32_t* offsets = reinterpret_cast<int32_t*>(base);
  base += align256((plan.counts + 1) * 4);
  int32_t* tmp = reinterpret_cast<int32_t*>(base);
  const size_t lds = static_cast<size_t>(nrows) * sizeof(int);
  const dim3 grid(plan.ntiles, a.Hkv);
  // With at most one tile per compute unit (long order-free tiles on the largest
  // problems), the count runs 1024 threads per tile so that 16 waves per compute unit
  // keep index loads in flight; otherwise 256.
  ZeroRanges z{};
  if (emit) z = ZeroRanges{emit->sb.counts, kKvSortZeroInts, reinterpret_cast<int32_t*>(emit->items),
                           4 * emit->max_items};
  if (static_cast<long long>(plan.ntiles) * a.Hkv <= device_cu_count())
    hipLaunchKernelGGL((csr_count_kernel<VARLEN, I32, 1024>), grid, dim3(1024), lds, stream, a,
                       plan.tile_q, plan.ntiles, counts, z);
  else
    hipLaunchKernelGGL((csr_count_kernel<VARLEN, I32, 256>), grid, dim3(256), lds, stream, a,
                       plan.tile_q, plan.ntiles, counts, z);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  err = launch_exclusive_scan(counts, offsets, plan.counts, tmp, stream);
  if (err != hipSuccess) return err;
  // The ordered scatter ranks with hash slots on tables wider than kCsrHashAboveRows,
  // else with per-row mask tables, where either fits the LDS (a workgroup may take up to
  // 160 KiB on gfx950; above 64 KiB the kernel must be allowed to), else with ballots.
  const size_t lds_cursors = 4 * static_cast<size_t>((nrows + 1) & ~1) * 4;
  const size_t lds_mask = lds_cursors + 4 * static_cast<size_t>(nrows) * 8;
  const size_t lds_hash = lds_cursors + 4 * kCsrHashSlots * (8 + 4);
  const auto allow = [](const void* kern, size_t bytes) {
    if (bytes <= 64 * 1024) return true;
    const bool ok = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                        static_cast<int>(bytes)) == hipSuccess;
    (void)hipGetLastError();  // a refused attribute leaves the next ranking
    return ok;
  };
  const bool hash_ok =
      ordered && nrows > kCsrHashAboveRows && lds_hash <= kCsrMaskLdsMax &&
      allow(reinterpret_cast<const void*>(&csr_scatter4_kernel<VARLEN, I32, kRankHash>), lds_hash);
  const bool mask_ok =
      ordered && !hash_ok && lds_mask <= kCsrMaskLdsMax &&
      allow(reinterpret_cast<const void*>(&csr_scatter4_kernel<VARLEN, I32, kRankMask>), lds_mask);
  if (hash_ok)
    hipLaunchKernelGGL((csr_scatter4_kernel<VARLEN, I32, kRankHash>), grid, dim3(256), lds_hash,
                       stream, a, plan.tile_q, plan.ntiles, offsets, q_idx, slot);
  else if (mask_ok)
    hipLaunchKernelGGL((csr_scatter4_kernel<VARLEN, I32, kRankMask>), grid, dim3(256), lds_mask,
                       stream, a, plan.tile_q, plan.ntiles, offsets, q_idx, slot);
  else if (ordered && 4 * lds <= 64 * 1024)  // within the default dynamic LDS limit
    hipLaunchKernelGGL((csr_scatter4_kernel<VARLEN, I32, kRankBallot>), grid, dim3(256), 4 * lds,
                       stream, a, plan.tile_q, plan.ntiles, offsets, q_idx, slot);
  else if (ordered)
    hipLaunchKernelGGL((csr_scatter_kernel<VARLEN, I32>), grid, dim3(64), lds, stream, a, plan.tile_q,
                       plan.ntiles, offsets, q_idx, slot);
  else if (flat && emit) {  // with the kv-centric items; LDS: cursors, row starts, keys
    const auto kern = &csr_scatter_unordered_kernel<VARLEN, I32, true, true>;
    const size_t lds_items = 2 * lds + kKvKeys * sizeof(int);
    if (lds_items > 64 * 1024) {
      const hipError_t ea = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                                hipFuncAttributeMaxDynamicSharedMemorySize,
                                                static_cast<int>(lds_items));
      if (ea != hipSuccess) return ea;
    }
    hipLaunchKernelGGL(kern, grid, dim3(256), lds_items, stream, a, plan.tile_q, plan.ntiles,
                       offsets, q_idx, slot, row_ptr, *emit);
  } else if (flat) {  // the order-free scatter also writes the row pointers (tile-0 blocks)
    hipLaunchKernelGGL((csr_scatter_unordered_kernel<VARLEN, I32, true, false>), grid, dim3(256),
                       lds, stream, a, plan.tile_q, plan.ntiles, offsets, q_idx, slot, row_ptr,
                       KvItemEmit{});
  } else {
    hipLaunchKernelGGL((csr_scatter_unordered_kernel<VARLEN, I32, false, false>), grid, dim3(256),
                       lds, stream, a, plan.tile_q, plan.ntiles, offsets, q_idx, slot, row_ptr,
                       KvItemEmit{});
  }
  if (ordered) {
    const long long nrp = static_cast<long long>(a.Hkv) * (nrows + 1);
    hipLaunchKernelGGL(csr_row_ptr_kernel, dim3(blocks_for(nrp, 256)), dim3(256), 0, stream,
                       offsets, a.Hkv, nrows, plan.ntiles, row_ptr);
  }
  return hipGetLastError();
}

template <bool VARLEN>
hipError_t build_csr(const CsrSrc& a, int32_t* row_ptr, int32_t* q_idx, int32_t* slot, void* ws,
                     hipStream_t stream, bool ordered, bool flat, const KvItemEmit* emit) {
  if (flat && (ordered || a.nq * a.topk >= (1LL << 31))) return hipErrorInvalidValue;
  if (emit && (!flat || emit->chunk_shift < 0 || emit->chunk_shift > 20)) return hipErrorInvalidValue;
  if (a.nq * a.topk < (1LL << 31))
    return build_csr_impl<VARLEN, true>(a, row_ptr, q_idx, slot, ws, stream, ordered, flat, emit);
  return build_csr_impl<VARLEN, false>(a, row_ptr, q_idx, slot, ws, stream, ordered, flat, emit);
}

}  // namespace

hipError_t launch_build_csr(const int32_t* q2k, int B, int Hkv, int Sq, int topk, int nblk,
                            int32_t* row_ptr, int32_t* q_idx, int32_t* slot, void* ws,
                            hipStream_t stream, bool ordered, bool flat, const KvItemEmit* emit) {
  CsrSrc a{};
  a.q2k = q2k;
  a.Hkv = Hkv; a.Sq = Sq; a.topk = topk; a.nblk = nblk;
  a.nrows = B * nblk;
  a.nq = static_cast<long long>(B) * Sq;
  return build_csr<false>(a, row_ptr, q_idx, slot, ws, stream, ordered, flat, emit);
}

hipError_t launch_build_csr_varlen(const int32_t* q2k, const VarlenTables& t, int Hkv,
                                   int total_q, int topk, int nrows, int32_t* row_ptr,
                                   int32_t* q_idx, int32_t* slot, void* ws, hipStream_t stream,
                                   bool ordered, bool flat, const KvItemEmit* emit) {
  CsrSrc a{};
  a.q2k = q2k;
  a.q_rows = t.q_rows;
  a.Hkv = Hkv; a.Sq = total_q; a.topk = topk; a.nblk = 0;
  a.nrows = nrows;
  a.nq = total_q;
  return build_csr<true>(a, row_ptr, q_idx, slot, ws, stream, ordered, flat, emit);
}

hipError_t launch_zero_ints(int32_t* p0, long long n0, int32_t* p1, long long n1,
                            hipStream_t stream) {
  if (n0 + n1 <= 0) return hipSuccess;
  const long long blocks = std::min<long long>((n0 + n1 + 255) / 256, 4096);
  hipLaunchKernelGGL(zero_ints_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0, stream,
                     p0, n0, p1, n1);
  return hipGetLastError();
}

}  // namespace msa
