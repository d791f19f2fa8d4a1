// Per-sequence tables of a variable-length batch (packed Q/K/V with
// cu_seqlens, the primary form of `sparse_atten_func` and `build_k2q_csr` on
// the page "MSA interface.py"). Sequence b's KV blocks are the CSR rows
// rowbase[b] .. rowbase[b+1]-1 with rowbase the prefix sum of ceil(Skv_b / 128)
// (the `total_rows` of the CSR); its block ids count from its first key. A paged
// batch gives every sequence max_pages rows (its page-table width).
//
// Two launches: one workgroup scans the per-sequence block counts (wave
// shuffles + a carry across 256-sequence rounds), then one thread per packed
// query / CSR row finds its sequence by binary search over cu_seqlens_q /
// rowbase and records what later kernels need of it (a query: the first CSR
// row and the block count of its sequence; a row: its sequence), so that no
// kernel searches per index entry.
#include "msa_internal.hpp"

namespace msa {

namespace {

__global__ __launch_bounds__(256) void varlen_rowbase_kernel(const int32_t* __restrict__ cu_k,
                                                             int B, long long total_k,
                                                             int blocks_per_seq,
                                                             int32_t* __restrict__ rowbase) {
  __shared__ long long wsum[4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long carry = 0;
  for (int base = 0; base < B; base += 256) {
    const int b = base + threadIdx.x;
    long long nb = 0;
    if (b < B && !cu_k) {
      nb = blocks_per_seq;
    } else if (b < B) {
      long long beg, len;
      seq_range(cu_k, b, total_k, beg, len);
      nb = (len + kBlk - 1) / kBlk;
    }
    long long x = nb;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long y = __shfl_up(x, d);
      if (lane >= d) x += y;
    }
    if (lane == 63) wsum[wave] = x;
    __syncthreads();
    long long before = carry, all = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wave) before += wsum[w];
      all += wsum[w];
    }
    if (b < B) rowbase[b] = static_cast<int32_t>(min(before + x - nb, 0x7FFFFFFFLL));
    carry += all;
    __syncthreads();
  }
  if (threadIdx.x == 0) rowbase[B] = static_cast<int32_t>(min(carry, 0x7FFFFFFFLL));
}

__global__ __launch_bounds__(256) void varlen_fill_kernel(const int32_t* __restrict__ cu_q,
                                                          const int32_t* __restrict__ rowbase,
                                                          int B, long long total_q, long long nrows,
                                                          int2* __restrict__ q_rows,
                                                          int32_t* __restrict__ row_seq) {
  const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < total_q) {
    const int b = seq_search(cu_q, B, i);
    q_rows[i] = make_int2(rowbase[b], rowbase[b + 1] - rowbase[b]);
  }
  if (row_seq && i < nrows) row_seq[i] = i < rowbase[B] ? seq_search(rowbase, B, i) : -1;
}

size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

}  // namespace

size_t varlen_tables_bytes(int B, long long total_q, long long nrows) {
  return align256((static_cast<size_t>(B) + 1) * 4) + align256(static_cast<size_t>(total_q) * 8) +
         align256(static_cast<size_t>(nrows) * 4);
}

VarlenTables varlen_tables_at(void* ws, int B, long long total_q, long long nrows) {
  char* p = static_cast<char*>(ws);
  VarlenTables t;
  t.rowbase = reinterpret_cast<int32_t*>(p);
  p += align256((static_cast<size_t>(B) + 1) * 4);
  t.q_rows = reinterpret_cast<int2*>(p);
  p += align256(static_cast<size_t>(total_q) * 8);
  t.row_seq = reinterpret_cast<int32_t*>(p);
  (void)nrows;
  return t;
}

hipError_t launch_varlen_tables(const int32_t* cu_q, const int32_t* cu_k, int B, long long total_q,
                                long long total_k, long long nrows, const VarlenTables& t,
                                hipStream_t stream, int blocks_per_seq) {
  if (B <= 0 || (!cu_k && blocks_per_seq <= 0)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(varlen_rowbase_kernel, dim3(1), dim3(256), 0, stream, cu_k, B, total_k,
                     blocks_per_seq, t.rowbase);
  const long long n = total_q > nrows ? total_q : nrows;
  if (n > 0) {
    const long long blocks = (n + 255) / 256;
    if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
    hipLaunchKernelGGL(varlen_fill_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                       stream, cu_q, t.rowbase, B, total_q, nrows, t.q_rows, t.row_seq);
  }
  return hipGetLastError();
}

}  // namespace msa
