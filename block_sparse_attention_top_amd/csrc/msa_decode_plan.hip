// Split-KV schedule and partial merge of the dense paged decode (q2k = None in
// `sparse_decode_atten_func` and the plan/run `SparseDecodePagedAttentionWrapper`
// on the page "MSA interface.py"; the schedule properties follow the decode
// schedule tests on the page "test_sparse_atten.py": per-sequence page counts,
// chunk counts, o_indptr advancing by (queries x chunks) rows per sequence,
// merge_indptr giving every query row its chunk count, work items = sum of
// chunk counts).
//
// The schedule is built on the device from seqused_k (no host sync): one
// workgroup scans the per-sequence chunk counts (wave shuffles, a carry across
// 256-sequence rounds), then one workgroup per sequence writes its work items
// and merge offsets. The merge is the log-sum-exp combine of a query row's
// chunk partials, for the sequences that took more than one chunk.
#include "msa_internal.hpp"

#include <math.h>

namespace msa {

namespace {

__global__ __launch_bounds__(256) void decode_schedule_kernel(const int32_t* __restrict__ seqused,
                                                              int B, int Sq, int max_pages,
                                                              int chunk_pages, int split,
                                                              DecodeSchedule s) {
  __shared__ long long wsum[2][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  long long carry_w = 0, carry_r = 0;  // work items, partial rows
  for (int base = 0; base < B; base += 256) {
    const int b = base + threadIdx.x;
    long long cnt = 0;
    if (b < B) {
      long long len = seqused[b];
      len = len < 0 ? 0 : (len > static_cast<long long>(max_pages) * kBlk
                               ? static_cast<long long>(max_pages) * kBlk : len);
      const long long pages = (len + kBlk - 1) / kBlk;
      cnt = split ? (pages + chunk_pages - 1) / chunk_pages : 1;
      if (cnt < 1) cnt = 1;  // a sequence without keys still writes (0, -inf)
      s.kv_pages[b] = static_cast<int32_t>(pages);
      s.counts[b] = static_cast<int32_t>(cnt);
    }
    long long xw = cnt, xr = cnt * Sq;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const long long yw = __shfl_up(xw, d), yr = __shfl_up(xr, d);
      if (lane >= d) {
        xw += yw;
        xr += yr;
      }
    }
    if (lane == 63) {
      wsum[0][wave] = xw;
      wsum[1][wave] = xr;
    }
    __syncthreads();
    long long bw = carry_w, br = carry_r, aw = 0, ar = 0;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (w < wave) {
        bw += wsum[0][w];
        br += wsum[1][w];
      }
      aw += wsum[0][w];
      ar += wsum[1][w];
    }
    if (b < B) {
      s.work_off[b] = static_cast<int32_t>(bw + xw - cnt);
      s.o_indptr[b] = static_cast<int32_t>(br + xr - cnt * Sq);
    }
    carry_w += aw;
    carry_r += ar;
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    s.o_indptr[B] = static_cast<int32_t>(carry_r);
    s.merge_indptr[static_cast<long long>(B) * Sq] = static_cast<int32_t>(carry_r);
    *s.work_count = static_cast<int32_t>(carry_w);
  }
}

// one workgroup per sequence
__global__ __launch_bounds__(256) void decode_items_kernel(int Sq, int chunk_pages,
                                                           DecodeSchedule s) {
  const int b = blockIdx.x;
  const int cnt = s.counts[b], pages = s.kv_pages[b], w0 = s.work_off[b], r0 = s.o_indptr[b];
  const int per = cnt > 1 ? chunk_pages : pages;  // pages per chunk
  for (int c = threadIdx.x; c < cnt; c += blockDim.x) {
    const int first = c * per;
    const int n = pages - first < per ? pages - first : per;
    s.items[w0 + c] = make_int4(b, c, first, n < 0 ? 0 : n);
  }
  for (int q = threadIdx.x; q < Sq; q += blockDim.x)
    s.merge_indptr[static_cast<long long>(b) * Sq + q] = r0 + q * cnt;
}

// thread = (query row, head, 8-dim chunk); rows of single-chunk sequences were
// written final by the decode kernel
__global__ __launch_bounds__(256) void merge_decode_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part,
    const float* __restrict__ lse_t_part, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ o_indptr, int B, int Sq, int Hq, uint16_t* __restrict__ o,
    float* __restrict__ lse, float* __restrict__ lse_t) {
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long long rows = static_cast<long long>(B) * Sq * Hq;
  if (idx >= rows * 16) return;
  const int dc = static_cast<int>(idx & 15);
  const long long rh = idx >> 4;  // (b, q, head)
  const int head = static_cast<int>(rh % Hq);
  const long long gq = rh / Hq;
  const int b = static_cast<int>(gq / Sq), q = static_cast<int>(gq % Sq);
  const int cnt = counts[b];
  if (cnt <= 1) return;
  const long long r0 = static_cast<long long>(o_indptr[b]) + static_cast<long long>(q) * cnt;
  float m = -INFINITY;
  for (int c = 0; c < cnt; ++c) m = fmaxf(m, lse_part[(r0 + c) * Hq + head]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (m != -INFINITY) {
    float sum = 0.f;
    for (int c = 0; c < cnt; ++c) sum += expf(lse_part[(r0 + c) * Hq + head] - m);
    L = m + logf(sum);
    for (int c = 0; c < cnt; ++c) {
      const float l = lse_part[(r0 + c) * Hq + head];
      if (l == -INFINITY) continue;  // a chunk that saw no key left its O unwritten
      const float wgt = expf(l - L);
      const float* src = o_part + ((r0 + c) * Hq + head) * kD + 8 * dc;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 e = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += wgt * a[i];
        acc[4 + i] += wgt * e[i];
      }
    }
  }
  const u32x4 out = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  *reinterpret_cast<u32x4*>(o + rh * kD + 8 * dc) = out;
  if (dc == 0) {
    const long long li = (static_cast<long long>(b) * Hq + head) * Sq + q;
    lse[li] = L;
    if (lse_t_part) {
      float mt = -INFINITY;
      for (int c = 0; c < cnt; ++c) mt = fmaxf(mt, lse_t_part[(r0 + c) * Hq + head]);
      float st = 0.f;
      if (mt != -INFINITY)
        for (int c = 0; c < cnt; ++c) st += expf(lse_t_part[(r0 + c) * Hq + head] - mt);
      lse_t[li] = mt == -INFINITY ? -INFINITY : mt + logf(st);
    }
  }
}

}  // namespace

hipError_t launch_decode_schedule(const int32_t* seqused, int B, int Sq, int max_pages,
                                  int chunk_pages, bool split, const DecodeSchedule& s,
                                  hipStream_t stream) {
  if (B <= 0 || Sq <= 0 || chunk_pages <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(decode_schedule_kernel, dim3(1), dim3(256), 0, stream, seqused, B, Sq,
                     max_pages, chunk_pages, split ? 1 : 0, s);
  hipLaunchKernelGGL(decode_items_kernel, dim3(B), dim3(256), 0, stream, Sq, chunk_pages, s);
  return hipGetLastError();
}

hipError_t launch_merge_decode(const float* o_part, const float* lse_part, const float* lse_t_part,
                               const int32_t* counts, const int32_t* o_indptr, int B, int Sq,
                               int Hq, uint16_t* o, float* lse, float* lse_t, hipStream_t stream) {
  const long long total = static_cast<long long>(B) * Sq * Hq * 16;
  const long long blocks = (total + 255) / 256;
  if (blocks <= 0) return hipSuccess;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(merge_decode_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, o_part, lse_part, lse_t_part, counts, o_indptr, B, Sq, Hq, o, lse,
                     lse_t);
  return hipGetLastError();
}

}  // namespace msa
