// Dense paged decode (q2k = None): every key of the sequence, split into the
// chunks of the device-built schedule.
//
// The operation is the paged attention of `sparse_attention_ref` on the page
// "MiniMax-AI/MSA python/fmha_sm100/cute/test_sparse_atten.py" with every block
// of the sequence selected (pool addressed through page_table as in
// `pack_paged_kv`, keys at or past seqused_k masked, bottom-right causal limit
// q + seqused_k - Sq), run as the dense decode of `sparse_decode_atten_func` /
// the plan/run decode wrapper on the page "MSA interface.py": each (sequence,
// chunk) writes a normalised fp32 partial (O, LSE) per (query, head), merged
// afterwards by log-sum-exp, or the final O and LSE when the sequence took a
// single chunk.
//
// Layout on gfx950. A workgroup (4 waves, two per CU) takes one (sequence,
// chunk, KV head) work item. The Sq x qpk (query, head) columns of the KV head
// (at most 128) are split 32 per wave, so every K/V fragment read from LDS
// serves 32 columns: S^T = K Q^T and O^T += V^T P^T run as
// v_mfma_f32_32x32x16_bf16 with Q and O in registers. The chunk's keys stream
// as 32-token sub-tiles (16 KiB of K and V) through a ring of four LDS stages
// filled by direct global->LDS loads, three sub-tiles in flight while one is
// consumed, one barrier per sub-tile. Rows are stored unpadded (256 B) with their
// 16-byte chunks XOR-swizzled by 4(r & 3) ^ ((r >> 2) & 3), which keeps both the
// 32-row K fragment reads and the transposed V reads free of bank conflicts.
// The load addresses are a scalar base per (page, sub-tile) plus loop-invariant
// 32-bit lane offsets, and masking runs only on sub-tiles that cross some
// column's causal limit, so the per-sub-tile vector work is the softmax itself.
//
// FP8 is the fp8 decode of those pages (Q, K and V fp8 e4m3fn; the unnormalised
// probabilities rounded to e4m3 before the P V product, the row sum kept
// unrounded, as the test page's dense decode reference states). Every fp8 value
// is exact in bf16 and every product of two of them exact in fp32, so the kernel
// keeps the bf16 matrix path: Q is widened once, the K/V sub-tiles (8 KiB of fp8)
// stream through a five-stage direct-to-LDS ring and one cooperative pass per
// sub-tile widens the next sub-tile into one of two swizzled bf16 buffers while
// the current one is consumed, and P is rounded to e4m3 and widened back.
#include "msa_internal.hpp"
#include "msa_lds.hpp"

#include <math.h>

namespace msa {

namespace {

constexpr int kSub = 32;              // tokens per sub-tile
constexpr int kRow = 256;             // bytes per K/V row in LDS (no padding)
constexpr int kTile = kSub * kRow;    // one sub-tile of K (or V): 8 KiB
constexpr int kCols = 128;            // (query, head) columns per workgroup
constexpr int kTile8 = kSub * kD;     // one fp8 sub-tile of K (or V): 4 KiB
constexpr int kStages8 = 5;           // fp8 ring depth

// 16-byte chunk c of LDS row r sits at chunk position c ^ swz(r) of that row
__device__ __forceinline__ int swz(int r) { return (4 * (r & 3)) ^ ((r >> 2) & 3); }

// 8 fp8 values -> 8 bf16 (exact)
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 w) {
  const u32x4 r = {fp8x2_to_bf16x2<false>(w[0]), fp8x2_to_bf16x2<true>(w[0]),
                   fp8x2_to_bf16x2<false>(w[1]), fp8x2_to_bf16x2<true>(w[1])};
  return as_bf16x8(r);
}

// (p0, p1) rounded to e4m3 (nearest, ties to even), widened back: a bf16 pair
__device__ __forceinline__ uint32_t e4m3_round_bf16x2(float p0, float p1) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  const s16x2 f8 = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, p0, p1, 1.0f, false);
  return fp8x2_to_bf16x2<false>(__builtin_bit_cast(uint32_t, f8));
}

template <bool TEMP, bool FP8>
__global__ __launch_bounds__(256, 2) void dense_decode_kernel(QcParams p) {
  __shared__ int upage[kDecMaxEntries];  // the chunk's page ids (an id outside the pool: -1)

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int hkv = static_cast<int>(blockIdx.x % p.Hkv);
  const long long w = blockIdx.x / p.Hkv;
  if (w >= *p.dec_work_count) return;  // padding past the schedule's items
  const int4 work = p.dec_items[w];    // (b, chunk, first page, pages)
  const int b = work.x, sp = work.y, npg = work.w;
  long long kvlen = p.seqused[b];
  kvlen = kvlen < 0 ? 0 : min(kvlen, static_cast<long long>(p.max_pages) * kBlk);
  // the chunk's keys [t0, t0 + ntok): every query sees a prefix of them
  const long long t0 = static_cast<long long>(work.z) * kBlk;
  const long long tend = min(kvlen, t0 + static_cast<long long>(npg) * kBlk);
  const int ntok = tend > t0 ? static_cast<int>(tend - t0) : 0;
  const int T = (ntok + kSub - 1) / kSub;  // sub-tiles

  for (int u = tid; u < npg; u += 256) {
    const int pg = p.page_table[static_cast<long long>(b) * p.max_pages + work.z + u];
    upage[u] = (pg >= 0 && pg < p.num_pages) ? pg : -1;
  }

  // column state: lane (n32, h32) = column n32 of this wave (row 32 wave + n32 of the
  // query-major Sq x qpk columns), k-half h32
  const int n32 = lane & 31, h32 = lane >> 5;
  const int col = 32 * wave + n32;
  const int q32 = col / p.qpk;
  const bool col_ok = q32 < p.Sq;
  const int head = hkv * p.qpk + col % p.qpk;
  // keys of the chunk visible to the column: [0, lim)
  int lim = ntok;
  if (col_ok && p.causal) {
    const long long e = q32 + kvlen - p.Sq + 1 - t0;
    lim = static_cast<int>(e < 0 ? 0 : (e < ntok ? e : ntok));
  }
  int wmin = lim;  // the wave's smallest limit: sub-tiles below it need no mask
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) wmin = min(wmin, __shfl_xor(wmin, d));
  wmin = __builtin_amdgcn_readfirstlane(wmin);

  bf16x8 qm[8];
  {
    const long long qoff =
        ((static_cast<long long>(b) * p.Sq + (col_ok ? q32 : 0)) * p.Hq + head) * kD + 8 * h32;
#pragma unroll
    for (int kq = 0; kq < 8; ++kq) {
      if (FP8) {
        u32x2 w = *reinterpret_cast<const u32x2*>(reinterpret_cast<const uint8_t*>(p.q) + qoff +
                                                  16 * kq);
        if (!col_ok) w = u32x2{0, 0};
        qm[kq] = fp8x8_to_bf16x8(w);
      } else {
        u32x4 v = *reinterpret_cast<const u32x4*>(p.q + qoff + 16 * kq);
        if (!col_ok) v = u32x4{0, 0, 0, 0};
        qm[kq] = as_bf16x8(v);
      }
    }
  }
  f32x16 om[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) om[dt] = f32x16{};
  // reference max in raw score units (both halves of a column agree) and half the
  // column's sums of 2^((s - m) c2) and, for the temperature LSE, 2^((s - m) c2 / T)
  float m_ref = -INFINITY, l_run = 0.f, lt_run = 0.f;
  const float c2 = p.scale_log2, c2t = c2 * p.inv_temp;
  const float c2m = TEMP ? c2 * fmaxf(1.f, p.inv_temp) : c2;

  // Direct loads of a sub-tile: each wave writes 4-row groups 2w and 2w+1 of K and
  // of V; lane l fills LDS row 4 grp + l / 16 at chunk position l % 16 with logical
  // chunk (l % 16) ^ swz(row). Rows past the chunk's last key read that key's row
  // (finite data whose probabilities are exactly zero).
  const int lrow = lane >> 4, lpos = lane & 15;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  uint32_t loff[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int r = 4 * (2 * wave + j) + lrow;
    loff[j] = r * kRow + 16 * (lpos ^ swz(r));
  }
  const int tail = ntok - kSub * (T - 1);  // keys in the last sub-tile (1..32)
  __syncthreads();                         // page list complete

  // scalar base of sub-tile t (page row 32 (t % 4) of the chunk's page t / 4)
  auto row_base = [&](int t) -> long long {
    int pg = __builtin_amdgcn_readfirstlane(upage[t >> 2]);
    pg = pg < 0 ? 0 : pg;  // an id outside the pool reads page 0 (in bounds), masked below
    return (static_cast<long long>(pg) * p.Hkv + hkv) * kBlk + kSub * (t & 3);
  };

  auto issue = [&](int t, uint8_t* buf) {
    const long long row0 = row_base(t);
    const uint8_t* kb = static_cast<const uint8_t*>(p.k) + row0 * kRow;
    const uint8_t* vb = static_cast<const uint8_t*>(p.v) + row0 * kRow;
    uint32_t o0 = loff[0], o1 = loff[1];
    if (t == T - 1 && tail < kSub) {  // wave-uniform
      const int r0 = 8 * wave + lrow, r1 = r0 + 4;
      o0 = min(r0, tail - 1) * kRow + 16 * (lpos ^ swz(r0));
      o1 = min(r1, tail - 1) * kRow + 16 * (lpos ^ swz(r1));
    }
    const uint32_t kd = lds_addr(buf), vd = kd + kTile;
    lds_load16_s(kb, o0, kd + 8 * wave_u * kRow);
    lds_load16_s(vb, o0, vd + 8 * wave_u * kRow);
    lds_load16_s(kb, o1, kd + (8 * wave_u + 4) * kRow);
    lds_load16_s(vb, o1, vd + (8 * wave_u + 4) * kRow);
  };

  // LDS lane offsets (bytes): K fragment = row n32, logical chunk 2 kq + h32 at
  // position (2 kq + h32) ^ swz(n32); transposed V reads of rows 16 kk + 4 h32 + rr
  // (+ 8), logical byte 64 dt + 32 (j16 & 1) + 8 cq, whose chunk's low two bits XOR
  // with h32 (h32 + 2) and high two bits with rr
  const int rr = (lane & 15) >> 2, cq = lane & 3, j16 = lane >> 4;
  const int koff = n32 * kRow + 16 * (h32 ^ swz(n32));
  const int vlo = (4 * h32 + rr) * kRow + 16 * ((2 * (j16 & 1) + (cq >> 1)) ^ h32) + 8 * (cq & 1);
  const int vhi =
      (4 * h32 + rr + 8) * kRow + 16 * ((2 * (j16 & 1) + (cq >> 1)) ^ (h32 + 2)) + 8 * (cq & 1);

  // Softmax of the 32 x 32 score tile (softmax_scale > 0, so the max of the raw
  // scores gives the max of the scaled ones). The reference max only moves when a
  // column's tile max exceeds it by more than 8 in log2 units (then every column of
  // the wave rescales its O and sums), so unnormalised probabilities stay <= 256
  // and the common sub-tile does no O rescale.
  auto compute = [&](int t, const uint8_t* buf) {
    if (upage[t >> 2] < 0) return;  // wave-uniform: a page outside the pool adds nothing
    const uint8_t* ks = buf;
    const uint8_t* vs = buf + kTile;
    f32x16 sacc = mfma32(as_bf16x8(*reinterpret_cast<const u32x4*>(ks + koff)), qm[0], f32x16{});
#pragma unroll
    for (int kq = 1; kq < 8; ++kq) {
      const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(ks + (koff ^ (32 * kq))));
      sacc = mfma32(a, qm[kq], sacc);
    }
    // lane (n32, h32) holds tokens 8 (i / 4) + 4 h32 + i % 4 of column n32
    if (kSub * t + kSub > wmin) {  // wave-uniform: some column's limit falls in here
      const int vis = lim - kSub * t;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (8 * (i >> 2) + 4 * h32 + (i & 3) >= vis) sacc[i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[i], sacc[i + 1]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    if (__any((mx - m_ref) * c2m > 8.f)) {
      const float m_new = fmaxf(m_ref, mx);
      const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * c2);
      l_run *= alpha;
      if (TEMP) lt_run *= m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * c2t);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) om[dt] *= alpha;
      m_ref = m_new;
    }
    const float nmc = -(m_ref == -INFINITY ? 0.f : m_ref) * c2;
    u32x4 pw[2];
    float ps = 0.f, pst = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p0 = fast_exp2(fmaf(sacc[2 * i], c2, nmc));
      const float p1 = fast_exp2(fmaf(sacc[2 * i + 1], c2, nmc));
      pw[i >> 2][i & 3] = FP8 ? e4m3_round_bf16x2(p0, p1) : pack_bf16x2(p0, p1);
      ps += p0 + p1;
      if (TEMP)
        pst += fast_exp2(fmaf(sacc[2 * i], c2t, nmc * p.inv_temp)) +
               fast_exp2(fmaf(sacc[2 * i + 1], c2t, nmc * p.inv_temp));
    }
    l_run += ps;
    if (TEMP) lt_run += pst;
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const bf16x8 pb = as_bf16x8(pw[kk]);
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int dx = 64 * (dt ^ rr);
        const i16x4 lo4 = lds_read_tr16(vs + 16 * kk * kRow + vlo + dx);
        const i16x4 hi4 = lds_read_tr16(vs + 16 * kk * kRow + vhi + dx);
        om[dt] = mfma32(cat_tr(lo4, hi4), pb, om[dt]);
      }
    }
  };

  if constexpr (!FP8) {
    // ring of four stages (K sub-tile at offset 0, V sub-tile at kTile); separate
    // arrays keep the stage buffers distinct objects
    __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kTile], st1[2 * kTile];
    __shared__ __attribute__((aligned(1024))) uint8_t st2[2 * kTile], st3[2 * kTile];
    // Ring of four stages: while stage t is consumed, stages t+1 and t+2 are in
    // flight and stage t+3 goes into the buffer that t-1 used (free once every wave
    // has passed this phase's barrier). Each wave issues 4 loads per stage, so "own
    // loads of stage t landed" is vmcnt <= 8; the barrier then makes every wave's
    // share visible. Stages past the end re-read the last sub-tile (in bounds) so
    // that every phase issues the same number of loads.
    if (T > 0) {
      issue(0, st0);
      issue(min(1, T - 1), st1);
      issue(min(2, T - 1), st2);
      int t = 0;
  #define MSA_DENSE_PHASE(cur, nxt)                              \
      {                                                          \
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8));         \
        __builtin_amdgcn_s_barrier();                            \
        issue(min(t + 3, T - 1), nxt);                           \
        compute(t, cur);                                         \
        if (++t >= T) break;                                     \
      }
      while (true) {
        MSA_DENSE_PHASE(st0, st3)
        MSA_DENSE_PHASE(st1, st0)
        MSA_DENSE_PHASE(st2, st1)
        MSA_DENSE_PHASE(st3, st2)
      }
  #undef MSA_DENSE_PHASE
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // no load outlives the loop
    }
  } else {
    // fp8 ring of five stages (K sub-tile at 0, V sub-tile at kTile8) and two bf16
    // buffers in the layout the compute reads
    __shared__ __attribute__((aligned(1024))) uint8_t ring8[kStages8 * 2 * kTile8];
    __shared__ __attribute__((aligned(1024))) uint8_t wide[2 * 2 * kTile];
    // direct loads of an fp8 sub-tile: wave w writes rows 8w .. 8w+7 of K and of V,
    // lane l row 8w + l / 8, 16-byte chunk l % 8, row-major without padding
    const int r8 = 8 * wave + (lane >> 3), c8 = lane & 7;
    const uint32_t loff8 = r8 * kD + 16 * c8;
    auto issue8 = [&](int t, int slot) {
      const long long row0 = row_base(t);
      const uint8_t* kb = static_cast<const uint8_t*>(p.k) + row0 * kD;
      const uint8_t* vb = static_cast<const uint8_t*>(p.v) + row0 * kD;
      uint32_t o = loff8;
      if (t == T - 1 && tail < kSub) o = min(r8, tail - 1) * kD + 16 * c8;  // wave-uniform branch
      const uint32_t kd = lds_addr(ring8) + slot * (2 * kTile8) + 8 * wave_u * kD;
      lds_load16_s(kb, o, kd);
      lds_load16_s(vb, o, kd + kTile8);
    };
    // widen ring slot `slot` into bf16 buffer `wb`: thread = (row tid / 8, 16 fp8 of
    // chunk tid % 8), written as logical bf16 chunks 2c and 2c + 1 of that row
    const int rw = tid >> 3, cw = tid & 7;
    const int wlo = rw * kRow + 16 * ((2 * cw) ^ swz(rw));
    const int whi = rw * kRow + 16 * ((2 * cw + 1) ^ swz(rw));
    auto widen = [&](int slot, int wb) {
      const uint8_t* src = ring8 + slot * (2 * kTile8) + rw * kD + 16 * cw;
      uint8_t* dst = wide + wb * (2 * kTile);
      u32x4 o2[2];
      fp8x16_to_bf16x16(*reinterpret_cast<const u32x4*>(src), o2);
      *reinterpret_cast<u32x4*>(dst + wlo) = o2[0];
      *reinterpret_cast<u32x4*>(dst + whi) = o2[1];
      fp8x16_to_bf16x16(*reinterpret_cast<const u32x4*>(src + kTile8), o2);
      *reinterpret_cast<u32x4*>(dst + kTile + wlo) = o2[0];
      *reinterpret_cast<u32x4*>(dst + kTile + whi) = o2[1];
    };
    // While sub-tile t is consumed from bf16 buffer t % 2, sub-tile t+1 is widened
    // into the other buffer and sub-tiles t+2 .. t+5 are in flight; sub-tile t+5 goes
    // into ring slot t % 5, whose sub-tile t was widened in the previous phase. Each
    // wave issues 2 loads per sub-tile, so "own loads of t+1 landed" is vmcnt <= 6;
    // the barrier then makes every wave's share visible and retires the previous
    // phase's widening and compute. Sub-tiles past the end re-read the last one.
    if (T > 0) {
#pragma unroll
      for (int s = 0; s < kStages8; ++s) issue8(min(s, T - 1), s);
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8));
      __builtin_amdgcn_s_barrier();
      widen(0, 0);
      int t = 0, slot_in = 0, slot_next = 1;  // slot_in = t % 5, slot_next = (t + 1) % 5
      while (true) {
        __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(6));
        __builtin_amdgcn_s_barrier();
        issue8(min(t + kStages8, T - 1), slot_in);
        if (t + 1 < T) widen(slot_next, (t + 1) & 1);
        compute(t, wide + (t & 1) * (2 * kTile));
        if (++t >= T) break;
        slot_in = slot_next;
        slot_next = slot_next == kStages8 - 1 ? 0 : slot_next + 1;
      }
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // no load outlives the loop
    }
  }

  // epilogue: lane (n32, h32) holds dims 32 dt + 8 (i / 4) + 4 h32 + i % 4 of its column
  const float ps = l_run + __shfl_xor(l_run, 32);
  const float pst = lt_run + __shfl_xor(lt_run, 32);
  if (!col_ok) return;
  const bool any = ps > 0.f;
  const float inv = any ? 1.f / ps : 0.f;
  const float lse_v = any ? fmaf(m_ref, c2, fast_log2(ps)) * kLn2 : -INFINITY;
  const float lset_v = any ? fmaf(m_ref, c2t, fast_log2(pst)) * kLn2 : -INFINITY;
  const int count = p.dec_counts[b];
  const long long grow = static_cast<long long>(b) * p.Sq + q32;
  if (count == 1) {
    uint16_t* orow = p.o + (grow * p.Hq + head) * kD + 4 * h32;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const u32x2 v = {pack_bf16x2(om[dt][4 * j] * inv, om[dt][4 * j + 1] * inv),
                         pack_bf16x2(om[dt][4 * j + 2] * inv, om[dt][4 * j + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * j) = v;
      }
    if (h32 == 0) {
      const long long li = (static_cast<long long>(b) * p.Hq + head) * p.Sq + q32;
      p.lse[li] = lse_v;
      if (TEMP) p.lse_t[li] = lset_v;
    }
  } else {
    // a chunk that saw no key of this column leaves its O partial unwritten: the
    // merge reads O only where the partial LSE is finite
    const long long prow =
        (static_cast<long long>(p.dec_o_indptr[b]) + static_cast<long long>(q32) * count + sp) *
            p.Hq + head;
    if (any) {
      float* orow = p.o_part + prow * kD + 4 * h32;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x4 v = {om[dt][4 * j] * inv, om[dt][4 * j + 1] * inv, om[dt][4 * j + 2] * inv,
                           om[dt][4 * j + 3] * inv};
          *reinterpret_cast<f32x4*>(orow + 32 * dt + 8 * j) = v;
        }
    }
    if (h32 == 0) {
      p.lse_part[prow] = lse_v;
      if (TEMP) p.lse_t_part[prow] = lset_v;
    }
  }
}

}  // namespace

// the union-decode kernel's dense mode (msa_decode.hip), for more than 128 columns
// (up to 4 * kMaxQPerWave queries)
hipError_t launch_dense_decode_grouped(const QcParams& p, int padded_work, hipStream_t stream);

// Sq * qpk <= 128 runs the 32-column kernel above
hipError_t launch_dense_decode(const QcParams& p, int padded_work, hipStream_t stream) {
  if (p.Sq * p.qpk > kCols) {
    if (p.kv_fp8) return hipErrorInvalidValue;  // the grouped kernel reads bf16 only
    return launch_dense_decode_grouped(p, padded_work, stream);
  }
  const long long items = static_cast<long long>(padded_work) * p.Hkv;
  if (items <= 0) return hipSuccess;
  if (items > 0x7FFFFFFFLL || p.Sq < 1) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(items));
  if (p.kv_fp8 && p.lse_t)
    hipLaunchKernelGGL((dense_decode_kernel<true, true>), grid, dim3(256), 0, stream, p);
  else if (p.kv_fp8)
    hipLaunchKernelGGL((dense_decode_kernel<false, true>), grid, dim3(256), 0, stream, p);
  else if (p.lse_t)
    hipLaunchKernelGGL((dense_decode_kernel<true, false>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((dense_decode_kernel<false, false>), grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace msa
