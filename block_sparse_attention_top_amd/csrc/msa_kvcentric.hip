// kv-centric sparse attention forward: per-KV-block partials driven by the
// k2q CSR, merged afterwards by the slot combine.
//
// This follows the structure of the pages' sparse forward: `sparse_atten_func`
// on the page "MSA interface.py" consumes the kv-block -> query CSR from
// `build_k2q_csr`, computes for each (KV block, queries that selected it) a
// block-local softmax and a partial output plus its LSE, and merges
// the partials of each query by log-sum-exp in a separate `combine` step (its
// split-K semantics are the `o_partial_dtype` branch of `sparse_attention_ref`
// on the page "test_sparse_atten.py"). Partials are bf16 (the pages' default
// partial dtype), indexed by the slot t of the index row, and left
// unnormalised: U = sum_j e^(s_j - M) V_j with the block's reference max M,
// stored beside (LSE of the block, M); the combine applies e^(M - LSE_total).
//
// An fp8 e4m3fn K/V cache (FP8) is widened exactly to bf16 while the block's
// tiles are staged into LDS; everything after runs on the same bf16 tiles.
//
// With a temperature-scaled LSE requested (TEMP), each block also gets the
// log-sum-exp of its scores divided by T, from a second sum of
// 2^((s - M) c / T) kept beside the softmax sum; the combine merges those by
// log-sum-exp like the ordinary LSE.
//
// A variable-length batch (packed Q/K/V with cu_seqlens) differs only in where
// a row's keys and queries live: row r is block r - rowbase[b] of sequence b
// (from the per-row sequence table), the block's keys start at cu_seqlens_k[b]
// and may end inside it, and the causal limit uses the sequence's own lengths.
//
// Layout on gfx950. A work item is (KV head, CSR row = (b, block), a chunk of
// up to `chunk_entries` CSR entries), listed in an item table by the schedule
// kernel. A workgroup of 4 waves stages the block's K and V tiles
// (128 x 128 bf16, padded rows) and the chunk's (query, slot) entries in LDS;
// two workgroups share a CU, so one wave's softmax (VALU) overlaps the other
// wave's matrix work on each SIMD, and one workgroup's tile load overlaps the
// other's compute. Each wave takes 32 gathered (query, head) rows at a time as
// the N = 32 columns of v_mfma_f32_32x32x16_bf16, Q rows loaded from HBM one
// step ahead: S^T = K Q^T (K fragments by ds_read_b128), a block-local softmax
// per lane column (two 64-token halves, online), O^T = V^T P^T (V fragments by
// the transposing ds_read_b64_tr_b16).
#include "msa_internal.hpp"
#include "msa_lds.hpp"

#include <math.h>

namespace msa {

namespace {

template <int QPK, bool TEMP, bool FP8>
__global__ __launch_bounds__(256, 2) void kvcentric_kernel(KvParams p) {
  constexpr int kEnt = kKvChunkRows / QPK < kKvMaxEntries ? kKvChunkRows / QPK : kKvMaxEntries;
  __shared__ __attribute__((aligned(16))) uint8_t ks[kBlk * kKStride];
  __shared__ __attribute__((aligned(16))) uint8_t vs[kBlk * kVStride];
  __shared__ int ent_q[kEnt];
  __shared__ int ent_t[kEnt];

  const int total = p.chunk_ptr[p.Hkv * p.nrows];
  const int w = blockIdx.x;
  if (w >= total) return;
  const int tid = threadIdx.x;
  const int4 item = p.items[w];
  const int hkv = item.x, r = item.y, e0 = item.z, ne = item.w;
  // the row's sequence b and block s; the sequence's first query and query
  // count, first key and key count
  int s;
  long long qbeg, sq_b, kbeg, kvlen;
  if (p.cu_q) {
    const int b = p.row_seq[r];
    if (b < 0) return;  // a row past the last sequence holds no entries
    s = r - p.rowbase[b];
    seq_range(p.cu_q, b, p.total_q, qbeg, sq_b);
    seq_range(p.cu_k, b, p.total_k, kbeg, kvlen);
  } else {
    const int b = r / p.nblk;
    s = r % p.nblk;
    qbeg = static_cast<long long>(b) * p.Sq;
    sq_b = p.Sq;
    kbeg = static_cast<long long>(b) * p.Skv;
    kvlen = p.Skv;
  }
  const long long blk0 = static_cast<long long>(s) * kBlk;

  // stage the chunk's entries and the block's K and V (128 tokens x 256 B each)
  for (int i = tid; i < ne; i += 256) {
    ent_q[i] = p.q_idx[hkv * p.cap + e0 + i];
    ent_t[i] = p.slot[hkv * p.cap + e0 + i];
  }
  {
    // rows past the sequence's last key re-read that key; they are masked out of S.
    // 16-byte loads of 8 bf16, or of 16 fp8 widened to two bf16 chunks (exact).
    constexpr int kEpc = FP8 ? 16 : 8;      // elements per load
    constexpr int kCpr = kD / kEpc;         // loads per row
    constexpr int kLpt = kBlk * kCpr / 256; // loads per thread
    constexpr int kEsz = FP8 ? 1 : 2;
    const char* kb = static_cast<const char*>(p.k);
    const char* vb = static_cast<const char*>(p.v);
    u32x4 rk[kLpt], rv[kLpt];
#pragma unroll
    for (int i = 0; i < kLpt; ++i) {
      const int ci = i * 256 + tid;
      const int row = ci / kCpr, c = ci % kCpr;
      const long long tok = kbeg + min(blk0 + row, kvlen - 1);
      const long long off = ((tok * p.Hkv + hkv) * kD + c * kEpc) * kEsz;
      rk[i] = *reinterpret_cast<const u32x4*>(kb + off);
      rv[i] = *reinterpret_cast<const u32x4*>(vb + off);
    }
#pragma unroll
    for (int i = 0; i < kLpt; ++i) {
      const int ci = i * 256 + tid;
      const int row = ci / kCpr, c = ci % kCpr;
      if (FP8) {
        u32x4 kw[2], vw[2];
        fp8x16_to_bf16x16(rk[i], kw);
        fp8x16_to_bf16x16(rv[i], vw);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          *reinterpret_cast<u32x4*>(ks + k_off(row, 2 * c + h2)) = kw[h2];
          *reinterpret_cast<u32x4*>(vs + v_off(row, 2 * c + h2)) = vw[h2];
        }
        continue;
      }
      *reinterpret_cast<u32x4*>(ks + k_off(row, c)) = rk[i];
      *reinterpret_cast<u32x4*>(vs + v_off(row, c)) = rv[i];
    }
  }
  __syncthreads();

  const int wave = tid >> 6, lane = tid & 63;
  const int n = lane & 31;   // row column of the 32x32 MFMA
  const int h = lane >> 5;   // k-half
  constexpr int EPW = 32 / QPK;  // CSR entries per wave step
  const int ent = n / QPK, head_i = n % QPK;
  const int head = hkv * QPK + head_i;
  const int j16 = lane >> 4, lq = lane & 15, rr = lq >> 2, cq = lq & 3;
  const long long lim_off = kvlen - sq_b;
  const long long kend = min(kvlen - blk0, static_cast<long long>(kBlk));  // keys of the block
  const int nsteps = (ne + EPW - 1) / EPW;
  const float c2 = p.scale_log2;
  const float c2t = c2 * p.inv_temp;
  // the reference max moves when exceeded by 8 / max(1, 1/T) in log2 units, so that
  // neither the softmax sum's nor the temperature sum's terms exceed 2^8
  const float c2m = TEMP ? c2 * fmaxf(1.f, p.inv_temp) : c2;
  // lane offsets inside the tiles: K fragment row n, chunk h; V transposed reads
  const int kbase0 = n * kKStride + h * 16;
  const int vbase0 = (4 * h + rr) * kVStride + 32 * (j16 & 1) + 8 * cq;

  struct Rows {
    bf16x8 q[8];
    int gq, t;
    bool ok;
  };
  auto fetch = [&](int step, Rows& R) {
    const int i = step * EPW + ent;
    R.ok = i < ne;
    const int ii = R.ok ? i : 0;
    R.gq = ent_q[ii];
    R.t = ent_t[ii];
    const uint16_t* qrow = p.q + (static_cast<long long>(R.gq) * p.Hq + head) * kD + 8 * h;
#pragma unroll
    for (int kq = 0; kq < 8; ++kq)
      R.q[kq] = as_bf16x8(*reinterpret_cast<const u32x4*>(qrow + 16 * kq));
  };

  // A step's partial is stored at the start of the wave's next step, ahead of that
  // step's Q loads. Vector memory loads and stores share one in-order counter on
  // gfx950 (vmcnt), so waiting for the Q rows never waits for stores issued after them.
  struct Pending {
    u32x4 v[8];          // 16-byte runs of the unnormalised partial, in store order
    uint16_t* ob;        // this lane's first 16-byte run
    long long prow;      // (query, slot, head) row of the block LSEs
    float lse_b, mnat, lse_t;
    bool ok;
  };
  Pending pend;
  pend.ok = false;
  auto flush = [&](const Pending& pd) {
#pragma unroll
    for (int k = 0; k < 8; ++k)
      // written once, read once by the combine: non-temporal
      __builtin_nontemporal_store(pd.v[k], reinterpret_cast<u32x4*>(pd.ob + (2 * k + h) * (QPK * 8)));
    if (h == 0) {
      p.lse_part[pd.prow] = make_float2(pd.lse_b, pd.mnat);
      if (TEMP) p.lse_t_part[pd.prow] = pd.lse_t;
    }
  };

  Rows rc, rn;
  int step = wave;
  if (step < nsteps) fetch(step, rc);
  for (; step < nsteps; step += 4) {
    // Every load and store still in flight here was issued a whole step ago. Waiting
    // for all of them explicitly (vmcnt(0), lgkmcnt(0)) leaves the compiler's wait-count
    // pass with nothing outstanding, so the conditional stores and Q loads below cannot
    // make it wait for the loads just issued before the first product.
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));
    if (pend.ok) flush(pend);
    if (step + 4 < nsteps) fetch(step + 4, rn);
    // The tile offsets are made opaque per step so that the K fragments are
    // re-read from LDS each step instead of being held in registers.
    int kbase = kbase0, vbase = vbase0;
    asm volatile("" : "+v"(kbase), "+v"(vbase));
    const long long qpos = rc.gq - qbeg;
    const long long lim = p.causal ? qpos + lim_off : (1LL << 62);
    const int vis = rc.ok ? static_cast<int>(max(min(lim - blk0 + 1, kend), -1LL)) : 0;
    const bool full = __all(vis >= kBlk);
    // Block-local softmax in two 64-token halves. The reference max m_ref is the
    // first half's row max; the second half only rescales (online softmax) when
    // its max exceeds m_ref by more than 8 in log2 units, so that unnormalised
    // probabilities stay <= 256. P is rounded to bf16 for the P V product; the
    // row sum is accumulated in fp32 (summing the bf16-rounded values instead
    // moves the LSE by up to ~1.4e-3 when a few keys dominate a row).
    float m_ref = -INFINITY, ps = 0.f;
    float pst = 0.f;  // TEMP: sum of 2^((s - m_ref) * c2 / T)
    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // S^T half (raw dot products): tokens 64*hf + 32*mt + 8*(i/4) + 4*h + i%4 of row n
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = f32x16{};
#pragma unroll
        for (int kq = 0; kq < 8; ++kq) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
              ks + kbase + (64 * hf + 32 * mt) * kKStride + 32 * kq));
          sacc[mt] = mfma32(a, rc.q[kq], sacc[mt]);
        }
      }
      if (!full) {
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int j = 64 * hf + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
            if (j >= vis) sacc[mt][i] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[mt][i], sacc[mt][i + 1]));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      if (hf == 0) {
        m_ref = mx;
      } else if (__any((mx - m_ref) * c2m > 8.f)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * c2);
        ps *= alpha;
        if (TEMP) pst *= m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * c2t);
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
        m_ref = m_new;
      }
      const float nmc = -(m_ref == -INFINITY ? 0.f : m_ref) * c2;
      uint32_t pk[2][8];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const float p0 = fast_exp2(fmaf(sacc[mt][2 * i], c2, nmc));
          const float p1 = fast_exp2(fmaf(sacc[mt][2 * i + 1], c2, nmc));
          pk[mt][i] = pack_bf16x2(p0, p1);
          ps += p0 + p1;
          if (TEMP)
            pst += fast_exp2(fmaf(sacc[mt][2 * i], c2t, nmc * p.inv_temp)) +
                   fast_exp2(fmaf(sacc[mt][2 * i + 1], c2t, nmc * p.inv_temp));
        }
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int mt = kk >> 1, i0 = 4 * (kk & 1);
        const u32x4 pw = {pk[mt][i0], pk[mt][i0 + 1], pk[mt][i0 + 2], pk[mt][i0 + 3]};
        const bf16x8 pb = as_bf16x8(pw);
        // rows 64*hf + 16*kk + 4*h + rr (+8), columns 32*dt + 16*(j16&1) + 4*cq .. +3
        const uint8_t* vrow = vs + vbase + (64 * hf + 16 * kk) * kVStride;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt) {
          const i16x4 lo4 = lds_read_tr16(vrow + 64 * dt);
          const i16x4 hi4 = lds_read_tr16(vrow + 8 * kVStride + 64 * dt);
          oacc[dt] = mfma32(cat_tr(lo4, hi4), pb, oacc[dt]);
        }
      }
    }
    ps += __shfl_xor(ps, 32);
    if (TEMP) pst += __shfl_xor(pst, 32);
    // lane (n, h) holds dims 32*dt + 8*q4 + 4*h .. +3 of row n (unnormalised) as
    // bf16 pairs. Swapping the odd-q4 half of lane h=0 with the even-q4 half of
    // lane h=1 (v_permlane32_swap) leaves each lane 16 contiguous bytes:
    // dims 32*dt + 16*pp + 8*h .. +7.
    uint32_t ow[4][4][2];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        ow[dt][q4][0] = pack_bf16x2(oacc[dt][4 * q4 + 0], oacc[dt][4 * q4 + 1]);
        ow[dt][q4][1] = pack_bf16x2(oacc[dt][4 * q4 + 2], oacc[dt][4 * q4 + 3]);
      }
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp)
#pragma unroll
        for (int w2 = 0; w2 < 2; ++w2) {
          const auto sw = __builtin_amdgcn_permlane32_swap(ow[dt][2 * pp][w2], ow[dt][2 * pp + 1][w2],
                                                           false, false);
          ow[dt][2 * pp][w2] = sw[0];
          ow[dt][2 * pp + 1][w2] = sw[1];
        }
    // Partial block of (query, slot, KV head): [dim chunk c][head][8 dims] with
    // c = dims / 8, so one store instruction writes QPK * 32 contiguous bytes per query.
    pend.ok = rc.ok;
    {
      const long long pblk = ((static_cast<long long>(rc.gq) * p.topk + rc.t) * p.Hkv + hkv);
      pend.ob = p.o_part + pblk * (QPK * kD) + head_i * 8;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int pp = 0; pp < 2; ++pp)
          pend.v[2 * dt + pp] = u32x4{ow[dt][2 * pp][0], ow[dt][2 * pp][1], ow[dt][2 * pp + 1][0],
                                      ow[dt][2 * pp + 1][1]};
      pend.prow = (static_cast<long long>(rc.gq) * p.topk + rc.t) * p.Hq + head;
      // both LSEs as one explicit fma of the same shape, so that T = 1 gives equal bits
      const float mr = m_ref == -INFINITY ? 0.f : m_ref;
      pend.mnat = mr * c2 * kLn2;
      pend.lse_b = ps > 0.f ? fmaf(fast_log2(ps), kLn2, pend.mnat) : -INFINITY;
      if (TEMP) {
        const float mnat_t = mr * c2t * kLn2;
        pend.lse_t = ps > 0.f ? fmaf(fast_log2(pst), kLn2, mnat_t) : -INFINITY;
      }
    }
    rc = rn;
  }
  if (pend.ok) flush(pend);
}

constexpr int kQueryBuckets = 256;  // = the block size of the passes below

__device__ __forceinline__ int item_bucket(const int4& it, const int32_t* q_idx, long long cap,
                                           long long nq) {
  const long long q = q_idx[it.x * cap + it.z];
  return static_cast<int>(min(q * kQueryBuckets / nq, static_cast<long long>(kQueryBuckets - 1)));
}

// items[c] = (hkv, row, first entry, entry count) for every chunk c of every row; with
// bucket_counts, each item is also counted in the query bucket of its first query (the
// first queries of 8 chunks loaded together, counts gathered per block in LDS).
__global__ __launch_bounds__(256) void kv_items_kernel(
    const int32_t* __restrict__ row_ptr, const int32_t* __restrict__ chunk_ptr, int Hkv, int nrows,
    int chunk_entries, int4* __restrict__ items, const int32_t* __restrict__ q_idx, long long cap,
    long long nq, int32_t* __restrict__ bucket_counts) {
  __shared__ int hist[kQueryBuckets];
  if (bucket_counts) {
    hist[threadIdx.x] = 0;
    __syncthreads();
  }
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (idx < static_cast<long long>(Hkv) * nrows) {
    const int hkv = static_cast<int>(idx / nrows), r = static_cast<int>(idx % nrows);
    const int32_t* rp = row_ptr + static_cast<long long>(hkv) * (nrows + 1);
    const int beg = rp[r], end = rp[r + 1];
    int c = chunk_ptr[idx];
    constexpr int kB = 8;
    for (int e0 = beg; e0 < end; e0 += kB * chunk_entries) {
      int q[kB];
      if (bucket_counts) {
#pragma unroll
        for (int k = 0; k < kB; ++k) {
          const int e = e0 + k * chunk_entries;
          q[k] = q_idx[hkv * cap + (e < end ? e : end - 1)];
        }
      }
#pragma unroll
      for (int k = 0; k < kB; ++k) {
        const int e = e0 + k * chunk_entries;
        if (e >= end) break;
        items[c++] = make_int4(hkv, r, e, min(chunk_entries, end - e));
        if (bucket_counts)
          atomicAdd(&hist[static_cast<int>(min(q[k] * kQueryBuckets / nq,
                                               static_cast<long long>(kQueryBuckets - 1)))], 1);
      }
    }
  }
  if (bucket_counts) {
    __syncthreads();
    const int n = hist[threadIdx.x];
    if (n) atomicAdd(&bucket_counts[threadIdx.x], n);
  }
}

// The item table reordered by the first query of each item: a counting sort over
// kQueryBuckets query ranges. With the CSR rows ascending in query, an item covers
// a narrow query range, and items that run together then gather Q rows from a small
// part of Q. Order inside a bucket is arbitrary: each item writes its own partials,
// so the results do not depend on it. The counts come from the item-table kernel
// (on counters the chunk schedule cleared); a scan and a scatter follow.
//
// Scatter of the items into bucket order: each block reserves a range of every bucket
// with one atomic on the running cursors (the scanned counts) and places its items
// there.
__global__ __launch_bounds__(kQueryBuckets) void kv_sort_scatter(
    const int4* __restrict__ items, const int32_t* __restrict__ chunk_ptr, int nchunk_rows,
    const int32_t* __restrict__ q_idx, long long cap, long long nq, int32_t* __restrict__ cursor,
    int4* __restrict__ out) {
  __shared__ int h[kQueryBuckets];
  __shared__ int base[kQueryBuckets];
  const int total = chunk_ptr[nchunk_rows];
  const int c = blockIdx.x * kQueryBuckets + threadIdx.x;
  h[threadIdx.x] = 0;
  __syncthreads();
  int4 it = make_int4(0, 0, 0, 0);
  int b = -1, rank = 0;
  if (c < total) {
    it = items[c];
    b = item_bucket(it, q_idx, cap, nq);
    rank = atomicAdd(&h[b], 1);
  }
  __syncthreads();
  const int n = h[threadIdx.x];
  base[threadIdx.x] = n ? atomicAdd(&cursor[threadIdx.x], n) : 0;
  __syncthreads();
  if (b >= 0) out[base[b] + rank] = it;
}

// exclusive scan of the bucket counts, in place (one block)
__global__ __launch_bounds__(kQueryBuckets) void kv_sort_scan(int32_t* __restrict__ counts) {
  __shared__ int v[kQueryBuckets];
  const int t = threadIdx.x;
  const int own = counts[t];
  v[t] = own;
  __syncthreads();
  for (int d = 1; d < kQueryBuckets; d <<= 1) {
    const int add = t >= d ? v[t - d] : 0;
    __syncthreads();
    v[t] += add;
    __syncthreads();
  }
  counts[t] = v[t] - own;
}

template <int QPK>
void kv_launch(const KvParams& p, dim3 grid, hipStream_t stream) {
  const dim3 blk(256);
  if (p.lse_t_part && p.kv_fp8)
    hipLaunchKernelGGL((kvcentric_kernel<QPK, true, true>), grid, blk, 0, stream, p);
  else if (p.lse_t_part)
    hipLaunchKernelGGL((kvcentric_kernel<QPK, true, false>), grid, blk, 0, stream, p);
  else if (p.kv_fp8)
    hipLaunchKernelGGL((kvcentric_kernel<QPK, false, true>), grid, blk, 0, stream, p);
  else
    hipLaunchKernelGGL((kvcentric_kernel<QPK, false, false>), grid, blk, 0, stream, p);
}

}  // namespace

hipError_t launch_kv_items(const int32_t* row_ptr, const int32_t* chunk_ptr, int Hkv, int nrows,
                           int chunk_entries, int4* items, hipStream_t stream,
                           const int32_t* q_idx, long long cap, long long nq,
                           int32_t* bucket_counts) {
  const long long n = static_cast<long long>(Hkv) * nrows;
  if (bucket_counts && nq <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_items_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0,
                     stream, row_ptr, chunk_ptr, Hkv, nrows, chunk_entries, items, q_idx, cap, nq,
                     bucket_counts);
  return hipGetLastError();
}

hipError_t launch_kv_items_by_query(const int4* items, const int32_t* chunk_ptr, int nchunk_rows,
                                    const int32_t* q_idx, long long cap, long long nq,
                                    long long max_items, int32_t* counts, int4* out,
                                    hipStream_t stream) {
  if (nq <= 0 || max_items <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((max_items + kQueryBuckets - 1) / kQueryBuckets));
  const dim3 blk(kQueryBuckets);
  hipLaunchKernelGGL(kv_sort_scan, dim3(1), blk, 0, stream, counts);
  hipLaunchKernelGGL(kv_sort_scatter, grid, blk, 0, stream, items, chunk_ptr, nchunk_rows, q_idx,
                     cap, nq, counts, out);
  return hipGetLastError();
}

hipError_t launch_kvcentric(const KvParams& p, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  if (p.chunk_entries * p.qpk > kKvChunkRows || p.chunk_entries > kKvMaxEntries)
    return hipErrorInvalidValue;
  const dim3 g(grid);
  switch (p.qpk) {
    case 1: kv_launch<1>(p, g, stream); break;
    case 2: kv_launch<2>(p, g, stream); break;
    case 4: kv_launch<4>(p, g, stream); break;
    case 8: kv_launch<8>(p, g, stream); break;
    case 16: kv_launch<16>(p, g, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
