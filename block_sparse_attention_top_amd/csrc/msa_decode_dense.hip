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
// unrounded, as the test page's dense decode reference states). It runs on the
// fp8 matrix cores: sub-tiles of 64 tokens (16 KiB of fp8 K and V, the same ring
// and stage size), S^T = K Q^T and O^T += V^T P^T as v_mfma_f32_32x32x64_f8f6f4
// (K fragments by ds_read_b128, V^T fragments by the transposing
// ds_read_b64_tr_b8), and P packed to e4m3 with the hardware's round-to-nearest-
// even conversion -- which is exactly the rounding the definition asks for.
// Rows of the fp8 tiles (128 B) hold 16-byte chunk c at position c ^ ((r >> 1) & 7),
// conflict-free for both fragment reads.
#include "msa_internal.hpp"
#include "msa_lds.hpp"

#include <math.h>

namespace msa {

namespace {

constexpr int kSub = 32;              // tokens per sub-tile
constexpr int kRow = 256;             // bytes per K/V row in LDS (no padding)
constexpr int kTile = kSub * kRow;    // one sub-tile of K (or V): 8 KiB
constexpr int kCols = 128;            // (query, head) columns per workgroup
constexpr int kSub8 = 64;             // tokens per fp8 sub-tile
constexpr int kTile8 = kSub8 * kD;    // one fp8 sub-tile of K (or V): 8 KiB

// fp8 tiles: 16-byte chunk c of row r (128 B) at chunk position c ^ swz8(r)
__device__ __forceinline__ int swz8(int r) { return (r >> 1) & 7; }

typedef int i32x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  // e4m3 x e4m3 (format code 0 for both), no block scales
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}
__device__ __forceinline__ i32x8 cat8(u32x4 lo, u32x4 hi) {
  const i32x8 r = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  return r;
}

// 16-byte chunk c of LDS row r sits at chunk position c ^ swz(r) of that row
__device__ __forceinline__ int swz(int r) { return (4 * (r & 3)) ^ ((r >> 2) & 3); }

// four probabilities rounded to e4m3 (nearest, ties to even) and packed, first in
// the lowest byte
__device__ __forceinline__ uint32_t e4m3x4(float p0, float p1, float p2, float p3) {
  typedef short s16x2 __attribute__((ext_vector_type(2)));
  s16x2 w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, p0, p1, 1.0f, false);
  w = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(w, p2, p3, 1.0f, true);
  return __builtin_bit_cast(uint32_t, w);
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
  constexpr int kSubT = FP8 ? kSub8 : kSub;  // tokens per sub-tile
  constexpr int kPerPage = kBlk / kSubT;     // sub-tiles per page
  const int T = (ntok + kSubT - 1) / kSubT;  // sub-tiles

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

  // Q as MFMA B fragments: bf16, lane (n32, h32) dims 16 kq + 8 h32 .. +7; fp8, dims
  // 64 kq + 32 h32 .. +31 (the byte order the K fragments use too)
  bf16x8 qm[FP8 ? 1 : 8];
  i32x8 qf[FP8 ? 2 : 1];
  {
    const long long qrow = (static_cast<long long>(b) * p.Sq + (col_ok ? q32 : 0)) * p.Hq + head;
    if constexpr (FP8) {
      const uint8_t* q8 = reinterpret_cast<const uint8_t*>(p.q) + qrow * kD + 32 * h32;
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        u32x4 lo = *reinterpret_cast<const u32x4*>(q8 + 64 * kq);
        u32x4 hi = *reinterpret_cast<const u32x4*>(q8 + 64 * kq + 16);
        if (!col_ok) lo = hi = u32x4{0, 0, 0, 0};
        qf[kq] = cat8(lo, hi);
      }
    } else {
      const uint16_t* qb = p.q + qrow * kD + 8 * h32;
#pragma unroll
      for (int kq = 0; kq < 8; ++kq) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qb + 16 * kq);
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
  const int tail = ntok - kSubT * (T - 1);  // keys in the last sub-tile (1..kSubT)
  __syncthreads();                         // page list complete

  // scalar base of sub-tile t (page row kSubT (t % kPerPage) of the chunk's page
  // t / kPerPage)
  auto row_base = [&](int t) -> long long {
    int pg = __builtin_amdgcn_readfirstlane(upage[t / kPerPage]);
    pg = pg < 0 ? 0 : pg;  // an id outside the pool reads page 0 (in bounds), masked below
    return (static_cast<long long>(pg) * p.Hkv + hkv) * kBlk + kSubT * (t % kPerPage);
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
    lds_load16_s_nt(kb, o0, kd + 8 * wave_u * kRow);
    lds_load16_s_nt(vb, o0, vd + 8 * wave_u * kRow);
    lds_load16_s_nt(kb, o1, kd + (8 * wave_u + 4) * kRow);
    lds_load16_s_nt(vb, o1, vd + (8 * wave_u + 4) * kRow);
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
      pw[i >> 2][i & 3] = pack_bf16x2(p0, p1);
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

  // fp8 sub-tiles (64 rows of 128 B for K and for V): wave w writes rows 16w .. 16w+15
  // of each, lane l row 16w + 8j + l / 8 at chunk position l % 8 with logical chunk
  // (l % 8) ^ swz8(row); past the chunk's last key the last key's row is read
  const int rw8 = 16 * wave + (lane >> 3), pw8 = lane & 7;
  uint32_t loff8[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) loff8[j] = (rw8 + 8 * j) * kD + 16 * (pw8 ^ swz8(rw8 + 8 * j));
  auto issue8 = [&](int t, uint8_t* buf) {
    const long long row0 = row_base(t);
    const uint8_t* kb = static_cast<const uint8_t*>(p.k) + row0 * kD;
    const uint8_t* vb = static_cast<const uint8_t*>(p.v) + row0 * kD;
    uint32_t o0 = loff8[0], o1 = loff8[1];
    if (t == T - 1 && tail < kSub8) {  // wave-uniform
      o0 = min(rw8, tail - 1) * kD + 16 * (pw8 ^ swz8(rw8));
      o1 = min(rw8 + 8, tail - 1) * kD + 16 * (pw8 ^ swz8(rw8 + 8));
    }
    const uint32_t kd = lds_addr(buf) + 16 * wave_u * kD, vd = kd + kTile8;
    lds_load16_s_nt(kb, o0, kd);
    lds_load16_s_nt(vb, o0, vd);
    lds_load16_s_nt(kb, o1, kd + 8 * kD);
    lds_load16_s_nt(vb, o1, vd + 8 * kD);
  };
  // fp8 fragment offsets. K (A of S^T = K Q^T, 32x32x64): lane (n32, h32) reads row
  // 32 tt + n32, dims 64 kq + 32 h32 .. +31 = logical chunks 4 kq + 2 h32 (+1). V^T (A of
  // O^T = V^T P^T) by ds_read_b64_tr_b8: in each 16-lane group g, lane pairs (2b, 2b+1)
  // address token row T0 + b at dims D0 and D0 + 8, so lane j receives dim D0 + j of the
  // 8 tokens T0 .. T0+7; read i covers tokens 16 i + 8 h .. +7 (the byte order P takes
  // below), D0 = 32 dt + 16 (g & 1).
  const int gq = lane >> 4, lq = lane & 15;
  auto compute8 = [&](int t, const uint8_t* buf) {
    if (upage[t / kPerPage] < 0) return;  // wave-uniform: a page outside the pool adds nothing
    const uint8_t* ks = buf;
    const uint8_t* vs = buf + kTile8;
    f32x16 sacc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const int r = 32 * tt + n32;
      const uint8_t* krow = ks + r * kD;
#pragma unroll
      for (int kq = 0; kq < 2; ++kq) {
        const int c = 4 * kq + 2 * h32;
        const u32x4 lo = *reinterpret_cast<const u32x4*>(krow + 16 * (c ^ swz8(r)));
        const u32x4 hi = *reinterpret_cast<const u32x4*>(krow + 16 * ((c + 1) ^ swz8(r)));
        sacc[tt] = mfma_f8(cat8(lo, hi), qf[kq], kq == 0 ? f32x16{} : sacc[tt]);
      }
    }
    // lane (n32, h32) holds tokens 32 tt + 8 (i / 4) + 4 h32 + i % 4 of column n32
    if (kSub8 * t + kSub8 > wmin) {  // wave-uniform: some column's limit falls in here
      const int vis = lim - kSub8 * t;
#pragma unroll
      for (int tt = 0; tt < 2; ++tt)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (32 * tt + 8 * (i >> 2) + 4 * h32 + (i & 3) >= vis) sacc[tt][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int i = 0; i < 16; i += 2) mx = fmaxf(mx, fmaxf(sacc[tt][i], sacc[tt][i + 1]));
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
    // P as e4m3: word q = 4 tt + i / 4 holds tokens 8 q + 4 h32 .. +3
    uint32_t pq[8];
    float ps = 0.f, pst = 0.f;
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        float pv[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = fast_exp2(fmaf(sacc[tt][4 * q4 + e], c2, nmc));
          ps += pv[e];
          if (TEMP) pst += fast_exp2(fmaf(sacc[tt][4 * q4 + e], c2t, nmc * p.inv_temp));
        }
        pq[4 * tt + q4] = e4m3x4(pv[0], pv[1], pv[2], pv[3]);
      }
    l_run += ps;
    if (TEMP) lt_run += pst;
    // swap word 2i + 1 of the low half-wave with word 2i of the high one: lane h then
    // holds tokens 16 i + 8 h .. +7 in words 2i, 2i+1 (the B fragment's byte order)
#pragma unroll
    for (int i2 = 0; i2 < 4; ++i2) {
      const auto sw = __builtin_amdgcn_permlane32_swap(pq[2 * i2], pq[2 * i2 + 1], false, false);
      pq[2 * i2] = sw[0];
      pq[2 * i2 + 1] = sw[1];
    }
    const i32x8 pb = {(int)pq[0], (int)pq[1], (int)pq[2], (int)pq[3],
                      (int)pq[4], (int)pq[5], (int)pq[6], (int)pq[7]};
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) {
      const int chunk = 2 * dt + (gq & 1);
      i32x8 a;
#pragma unroll
      for (int i2 = 0; i2 < 4; ++i2) {
        const int row = 16 * i2 + 8 * (gq >> 1) + (lq >> 1);
        typedef int i32x2 __attribute__((ext_vector_type(2)));
        const i32x2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
            (__attribute__((address_space(3))) i32x2*)(vs + row * kD +
                                                       16 * (chunk ^ swz8(row)) + 8 * (lq & 1)));
        a[2 * i2] = v[0];
        a[2 * i2 + 1] = v[1];
      }
      om[dt] = mfma_f8(a, pb, om[dt]);
    }
  };

  // ring of four stages (K sub-tile at offset 0, V sub-tile at kTile (bf16) or kTile8
  // (fp8); 16 KiB either way); separate arrays keep the stage buffers distinct objects
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kTile], st1[2 * kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[2 * kTile], st3[2 * kTile];
  auto issue_t = [&](int t, uint8_t* buf) {
    if constexpr (FP8) issue8(t, buf); else issue(t, buf);
  };
  auto compute_t = [&](int t, const uint8_t* buf) {
    if constexpr (FP8) compute8(t, buf); else compute(t, buf);
  };
  // Ring of four stages: while stage t is consumed, stages t+1 and t+2 are in
  // flight and stage t+3 goes into the buffer that t-1 used (free once every wave
  // has passed this phase's barrier). Each wave issues 4 loads per stage, so "own
  // loads of stage t landed" is vmcnt <= 8; the barrier then makes every wave's
  // share visible. Stages past the end re-read the last sub-tile (in bounds) so
  // that every phase issues the same number of loads.
  if (T > 0) {
    issue_t(0, st0);
    issue_t(min(1, T - 1), st1);
    issue_t(min(2, T - 1), st2);
    int t = 0;
#define MSA_DENSE_PHASE(cur, nxt)                              \
    {                                                          \
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8));         \
      __builtin_amdgcn_s_barrier();                            \
      issue_t(min(t + 3, T - 1), nxt);                         \
      compute_t(t, cur);                                       \
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
