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
// A paged K/V cache (PAGED) differs only in where a block's keys live: block s of
// sequence b is one page of the pools, page_table[b][s], and the sequence's keys end
// at seqused[b]; its queries are uniform (b * Sq ..) or packed (cu_seqlens_q, with
// max_pages CSR rows per sequence). A block past those keys, or whose page id is outside the pools,
// contributes nothing (its partials are empty and nothing of it is read), as on the
// paged q-centric kernel.
//
// Layout on gfx950. A work item is (KV head, CSR row = (b, block), a chunk of
// up to `chunk_entries` CSR entries), listed in an item table by the CSR scatter
// (or kv_items_kernel for a caller's CSR) and ordered by (KV head, first query) into
// one stream per KV head (see kvcentric_kernel). A workgroup of 4 waves stages the block's K and V tiles
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

#include <algorithm>

namespace msa {

namespace {

template <int QPK>
constexpr int kv_item_entries() {
  return kKvChunkRows / QPK < kKvMaxEntries ? kKvChunkRows / QPK : kKvMaxEntries;
}

// One work item: stage the block's K/V tiles and the chunk's entries in LDS, then
// each wave computes the partials of 32 gathered (query, head) rows per step.
template <int QPK, bool TEMP, bool FP8, bool PAGED>
__device__ __forceinline__ void kv_item(const KvParams& p, const int4 item, uint8_t* ks,
                                        uint8_t* vs, int* ent_q, int* ent_t) {
  const int tid = threadIdx.x;
  const int hkv = item.x, r = item.y, e0 = item.z, ne = item.w;
  // the row's sequence b and block s; the sequence's first query and query
  // count, first key and key count
  int s;
  long long qbeg, sq_b, kbeg, kvlen;
  int page = 0;       // PAGED: the block's page
  bool dead = false;  // PAGED: the block has no keys to read (past seqused, or a bad page)
  if (PAGED) {
    int b;
    if (p.cu_q) {  // packed queries: rows rowbase[b] .. + nblk are sequence b's blocks
      b = p.row_seq[r];
      if (b < 0) return;
      s = r - p.rowbase[b];
      seq_range(p.cu_q, b, p.total_q, qbeg, sq_b);
    } else {
      b = r / p.nblk;
      s = r % p.nblk;
      qbeg = static_cast<long long>(b) * p.Sq;
      sq_b = p.Sq;
    }
    kbeg = 0;
    kvlen = p.seqused[b];
    if (static_cast<long long>(s) * kBlk < kvlen)
      page = p.page_table[static_cast<long long>(b) * p.nblk + s];
    dead = !(static_cast<long long>(s) * kBlk < kvlen && page >= 0 && page < p.num_pages);
    if (dead) page = 0;
  } else if (p.cu_q) {
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
  if (p.slot) {
    // a caller's CSR: an entry whose query is not in the row's sequence or whose slot
    // is outside [0, topk) is kept as padding (slot -1, query 0: nothing gathered out
    // of bounds, nothing stored)
    for (int i = tid; i < ne; i += 256) {
      const int q = p.q_idx[hkv * p.cap + e0 + i];
      const int t = p.slot[hkv * p.cap + e0 + i];
      const bool v = q >= qbeg && q < qbeg + sq_b && t >= 0 && t < p.topk;
      ent_q[i] = v ? q : 0;
      ent_t[i] = v ? t : -1;
    }
  } else {  // entries stored as index-table positions query * topk + slot
    for (int i = tid; i < ne; i += 256) {
      const int e = p.q_idx[hkv * p.cap + e0 + i];
      const int q = static_cast<int>(static_cast<uint32_t>(e) / static_cast<uint32_t>(p.topk));
      ent_q[i] = q;
      ent_t[i] = e - q * p.topk;
    }
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
      if (PAGED) {
        // a dead block's tiles are zeros: its keys are all masked, and P V must not
        // meet non-finite values
        if (dead) {
          rk[i] = rv[i] = u32x4{0, 0, 0, 0};
          continue;
        }
        const long long j = min(blk0 + row, kvlen - 1) - blk0;  // in [0, 128): same page
        const long long off =
            (((static_cast<long long>(page) * p.Hkv + hkv) * kBlk + j) * kD + c * kEpc) * kEsz;
        rk[i] = *reinterpret_cast<const u32x4*>(kb + off);
        rv[i] = *reinterpret_cast<const u32x4*>(vb + off);
        continue;
      }
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
  // keys of the block (none for a dead one)
  const long long kend = PAGED && dead ? 0 : min(kvlen - blk0, static_cast<long long>(kBlk));
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
    const int ii = i < ne ? i : 0;
    R.gq = ent_q[ii];
    R.t = ent_t[ii];
    R.ok = i < ne && R.t >= 0;
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
      } else {
        // The rescale is decided per row: a row moves its reference max only when its
        // own second half exceeds it by the gap, and every other row keeps it and
        // multiplies by exactly 1. A row's result then depends on its own scores
        // alone, not on which rows share its wave step (the library's own CSR is
        // order-free, so that grouping changes from call to call).
        const bool resc = (mx - m_ref) * c2m > 8.f;
        if (__any(resc)) {
          const float m_new = resc ? mx : m_ref;
          const float alpha =
              !resc ? 1.f : m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * c2);
          ps *= alpha;
          if (TEMP)
            pst *= !resc ? 1.f : m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * c2t);
#pragma unroll
          for (int dt = 0; dt < 4; ++dt) oacc[dt] *= alpha;
          m_ref = m_new;
        }
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

// Persistent kv-centric kernel. The item table is ordered by key (KV head, first
// query) and cut into p.streams streams of equal key ranges, so that a stream is the
// items of one KV head (or of one query range of it) in query order. Workgroups are
// dealt round-robin over the 8 XCDs, so team blockIdx % p.streams runs on the same
// XCDs throughout; it takes the items of its own stream first, in order, through
// the stream's counter, so that the items running together on an XCD gather Q rows
// from one narrow query range of one KV head, which its L2 keeps. A workgroup whose
// stream is exhausted moves on to the next stream. Every item is taken exactly once
// (one atomic per take), no workgroup waits for another, and each workgroup stops
// after finding all streams exhausted.
//
// With the temperature-scaled LSE (TEMP) the kernel takes one item per workgroup
// instead (grid = the item bound; a workgroup exits once every stream is exhausted):
// its second running sum and LSE make the item loop spill (132-180 bytes per lane),
// and one item per workgroup measured 8% faster there (8192 causal queries, 64 query
// heads over 4 KV heads, T = 2), while the loop is 1-3.5% faster without it.
template <bool TEMP>
constexpr bool kv_persistent() {
  return !TEMP;
}
template <int QPK, bool TEMP, bool FP8, bool PAGED>
__global__ __launch_bounds__(256, 2) void kvcentric_kernel(KvParams p) {
  constexpr int kEnt = kv_item_entries<QPK>();
  __shared__ __attribute__((aligned(16))) uint8_t ks[kBlk * kKStride];
  __shared__ __attribute__((aligned(16))) uint8_t vs[kBlk * kVStride];
  __shared__ int ent_q[kEnt];
  __shared__ int ent_t[kEnt];
  __shared__ int s_item;
  const int nst = p.streams;  // 1, 2, 4 or 8: divides kKvStreams
  const int keys_per_stream = kKvKeys / nst;
  const int team = blockIdx.x % nst;
  int tried = 0;  // streams found exhausted (thread 0)
  for (;;) {
    if (threadIdx.x == 0) {
      int got = -1;
      while (tried < nst) {
        const int st = (team + tried) % nst;
        const int beg = p.key_start[st * keys_per_stream];
        const int end = p.key_start[(st + 1) * keys_per_stream];
        if (beg < end) {
          const int i = atomicAdd(&p.stream_next[st], 1);
          if (i < end - beg) {
            got = beg + i;
            break;
          }
        }
        ++tried;
      }
      s_item = got;
    }
    __syncthreads();
    const int w = s_item;
    if (w < 0) break;
    kv_item<QPK, TEMP, FP8, PAGED>(p, p.items[w], ks, vs, ent_q, ent_t);
    if constexpr (!kv_persistent<TEMP>()) break;
    __syncthreads();  // LDS tiles and s_item are reused by the next item
  }
}

// items for the chunks of 2^chunk_shift entries of every row of a caller's CSR, each
// at its slot (kv_item_slot), and the per-key item counts (counts gathered per
// workgroup in LDS). One wave per (KV head, row): lane l writes the row's chunks l,
// l + 64, ..., so that a long row is spread over a wave and every first-query load of
// a round is in flight together. The order-free CSR that the library builds itself
// lists its items while it scatters (KvItemEmit), so this kernel runs only for a
// caller's CSR. Its row_ptr is not trusted: a row is used only if kv_row_ok, which
// keeps every read and slot in bounds; any other row raises sb.bad, and the sort then
// places no item at all (with a row out of order, rows may overlap, their slots collide
// and the counts overshoot).
__global__ __launch_bounds__(256) void kv_items_kernel(
    const int32_t* __restrict__ row_ptr, int Hkv, int nrows, int chunk_shift, long long per_head,
    int4* __restrict__ items, const int32_t* __restrict__ q_idx, long long cap, long long nq,
    int qdiv, KvSortBuffers sb) {
  __shared__ int hist[kKvKeys];
  for (int i = threadIdx.x; i < kKvKeys; i += 256) hist[i] = 0;
  __syncthreads();
  const long long idx = static_cast<long long>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int chunk = 1 << chunk_shift;
  if (idx < static_cast<long long>(Hkv) * nrows) {
    const int hkv = static_cast<int>(idx / nrows), r = static_cast<int>(idx % nrows);
    const int32_t* rp = row_ptr + static_cast<long long>(hkv) * (nrows + 1);
    const int rb = rp[r], re = rp[r + 1];
    const bool ok = kv_row_ok(rb, re, cap);
    if (!ok && lane == 0) atomicOr(sb.bad, 1);
    const int beg = ok ? rb : 0, end = ok ? re : 0;
    const int nch = end > beg ? (end - beg + chunk - 1) >> chunk_shift : 0;
    for (int j = lane; j < nch; j += 64) {
      const int e = beg + j * chunk;
      const int q = q_idx[hkv * cap + e] / qdiv;
      items[kv_item_slot(hkv, per_head, e, chunk_shift, r)] =
          make_int4(hkv, r, e, min(chunk, end - e));
      atomicAdd(&hist[kv_item_key(hkv, q, nq, Hkv)], 1);
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < kKvKeys; i += 256) {
    const int n = hist[i];
    if (n) atomicAdd(&sb.counts[i], n);
  }
}

// The item table in key order (a counting sort). Every workgroup scans the key counts
// itself (8 keys per thread), so no separate scan launch is needed; workgroup 0
// publishes the starts in sb.key_start (key_start[kKvKeys] = the item count) for the
// forward kernel. Each workgroup then ranks the items of its 256 table slots (unused
// slots hold entry count 0) per key in LDS, reserves a range of every key it holds
// with one atomic on the key's cursor, and places its items there. Order inside a key
// is arbitrary: each item writes its own partials, so the results do not depend on it.
// With sb.bad set every count reads as zero: no item is placed and the starts are 0.
__global__ __launch_bounds__(256) void kv_sort_scatter(
    const int4* __restrict__ items, long long nslots, KvSortBuffers sb, int Hkv,
    const int32_t* __restrict__ q_idx, long long cap, long long nq, int qdiv,
    int4* __restrict__ out) {
  constexpr int kPer = kKvKeys / 256;
  __shared__ int h[kKvKeys];
  __shared__ int base[kKvKeys];
  __shared__ int wsum[4];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  // a caller's CSR whose row_ptr failed the item kernel's check: no items at all
  const bool bad = *sb.bad != 0;
  int c[kPer], own = 0;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    c[k] = bad ? 0 : sb.counts[t * kPer + k];
    own += c[k];
  }
  int x = own;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(x, d);
    if (lane >= d) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  for (int i = t; i < kKvKeys; i += 256) h[i] = 0;
  __syncthreads();
  int before = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) before += w < wave ? wsum[w] : 0;
  int run = before + x - own;
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    base[t * kPer + k] = run;
    if (blockIdx.x == 0) sb.key_start[t * kPer + k] = run;
    run += c[k];
  }
  if (t == 255 && blockIdx.x == 0) sb.key_start[kKvKeys] = run;
  __syncthreads();
  const long long ci = static_cast<long long>(blockIdx.x) * 256 + t;
  int4 it = make_int4(0, 0, 0, 0);
  int key = -1, rank = 0;
  if (ci < nslots && !bad) {
    it = items[ci];
    if (it.w > 0) {
      key = kv_item_key(it.x, q_idx[it.x * cap + it.z] / qdiv, nq, Hkv);
      rank = atomicAdd(&h[key], 1);
    }
  }
  __syncthreads();
  for (int i = t; i < kKvKeys; i += 256) {
    const int n = h[i];
    if (n) base[i] += atomicAdd(&sb.cursor[i], n);
  }
  __syncthreads();
  if (key >= 0) out[base[key] + rank] = it;
}

template <int QPK, bool PAGED>
void kv_launch(const KvParams& p, long long max_items, hipStream_t stream) {
  const dim3 blk(256);
  // persistent: two workgroups per compute unit (the kernel's occupancy), at most one
  // per item; otherwise one workgroup per item
  const bool persistent = p.lse_t_part ? kv_persistent<true>() : kv_persistent<false>();
  const dim3 grid(static_cast<unsigned>(
      persistent ? std::min<long long>(max_items, 2LL * device_cu_count()) : max_items));
  if (p.lse_t_part && p.kv_fp8)
    hipLaunchKernelGGL((kvcentric_kernel<QPK, true, true, PAGED>), grid, blk, 0, stream, p);
  else if (p.lse_t_part)
    hipLaunchKernelGGL((kvcentric_kernel<QPK, true, false, PAGED>), grid, blk, 0, stream, p);
  else if (p.kv_fp8)
    hipLaunchKernelGGL((kvcentric_kernel<QPK, false, true, PAGED>), grid, blk, 0, stream, p);
  else
    hipLaunchKernelGGL((kvcentric_kernel<QPK, false, false, PAGED>), grid, blk, 0, stream, p);
}
template <bool PAGED>
hipError_t kv_launch_qpk(const KvParams& p, long long max_items, hipStream_t stream) {
  switch (p.qpk) {
    case 1: kv_launch<1, PAGED>(p, max_items, stream); break;
    case 2: kv_launch<2, PAGED>(p, max_items, stream); break;
    case 4: kv_launch<4, PAGED>(p, max_items, stream); break;
    case 8: kv_launch<8, PAGED>(p, max_items, stream); break;
    case 16: kv_launch<16, PAGED>(p, max_items, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_items(const int32_t* row_ptr, int Hkv, int nrows, int chunk_shift,
                           long long per_head, int4* items, const int32_t* q_idx, long long cap,
                           long long nq, int qdiv, const KvSortBuffers& sb, hipStream_t stream) {
  const long long n = static_cast<long long>(Hkv) * nrows;
  if (nq <= 0 || n <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(kv_items_kernel, dim3(static_cast<unsigned>((n + 3) / 4)), dim3(256), 0,
                     stream, row_ptr, Hkv, nrows, chunk_shift, per_head, items, q_idx, cap, nq,
                     qdiv, sb);
  return hipGetLastError();
}

hipError_t launch_kv_items_by_key(const int4* items, int Hkv, const int32_t* q_idx, long long cap,
                                  long long nq, int qdiv, long long max_items,
                                  const KvSortBuffers& sb, int4* out, hipStream_t stream) {
  if (nq <= 0 || max_items <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>((max_items + 255) / 256));
  hipLaunchKernelGGL(kv_sort_scatter, grid, dim3(256), 0, stream, items, max_items, sb, Hkv, q_idx,
                     cap, nq, qdiv, out);
  return hipGetLastError();
}

hipError_t launch_kvcentric(const KvParams& p, long long max_items, hipStream_t stream) {
  if (max_items <= 0) return hipSuccess;
  if (max_items > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (p.chunk_entries * p.qpk > kKvChunkRows || p.chunk_entries > kKvMaxEntries)
    return hipErrorInvalidValue;
  if (p.page_table && (!p.seqused || p.num_pages <= 0 || p.nblk <= 0)) return hipErrorInvalidValue;
  return p.page_table ? kv_launch_qpk<true>(p, max_items, stream)
                      : kv_launch_qpk<false>(p, max_items, stream);
}

}  // namespace msa
