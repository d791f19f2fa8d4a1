// q-centric fused sparse attention forward (one wave per index row).
//
// The operation is the sparse attention of `sparse_attention_ref` on the page
// "MiniMax-AI/MSA python/fmha_sm100/cute/test_sparse_atten.py": for query
// (b, q) and KV head hkv, the qhead_per_kv query heads that share the index
// row q2k[b][hkv][q][:] attend to the union of its valid blocks, masked by
// seqused_k (paged) and the bottom-right causal limit q + kvlen - Sq, with a
// natural-log LSE and (O = 0, LSE = -inf) for an empty key set.
//
// Layout on gfx950: a workgroup of one or two waves takes one index row (or one
// split of it); with two, wave w streams slots w, w + 2, ... with its own online
// softmax and LDS tiles, and the two states are merged by log-sum-exp at the end
// (twice the waves in flight without a separate combine pass). Within a wave, the qpk
// heads of the row are the N = 16 columns of
// v_mfma_f32_16x16x32_bf16 (zero-padded when qpk < 16). Each selected block
// is streamed as four 32-token sub-tiles: K and V are fetched with 16-byte
// loads into registers one sub-tile ahead, stored to LDS (padded rows), and
// consumed as S^T = K Q^T (K fragments by ds_read_b128) and
// O^T += V^T P^T (V fragments by the transposing ds_read_b64_tr_b16), so each
// head's softmax statistics stay in its own lane column. Online softmax in
// fp32 with exp2 and the scale folded into log2 units.
//
// With splits > 1 a wave handles a contiguous share of the slots and writes a
// normalised fp32 partial (O, LSE) that the split combine merges (the
// split-KV decode of `sparse_decode_atten_func` on the page "MSA interface.py").
//
// With an fp8 e4m3fn K/V cache (FP8) each 16-byte load brings 16 elements, which
// are widened exactly to bf16 (v_cvt_scalef32_pk_bf16_fp8) while being stored to
// LDS, so the products run on the same bf16 tiles.
//
// The temperature-scaled LSE (TEMP) keeps a second running sum of
// 2^((x - m) / T) next to the softmax sum; the running max needs no second copy
// because max(x / T) = max(x) / T for T > 0.
//
// Variable-length batches (packed Q/K/V with cu_seqlens, contiguous K/V): a
// wave finds the sequence of its query row by binary search over
// cu_seqlens_q; block ids count from the sequence's first key and the causal
// limit uses the sequence's own lengths.
#include "msa_internal.hpp"

#include <math.h>

namespace msa {

namespace {

constexpr int kSub = 32;  // tokens per sub-tile

// Orders one wave's LDS accesses for the compiler (the hardware keeps a wave's LDS
// operations in order); each wave stages and reads only its own tiles.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// kWaves waves per index row (or split), each taking every kWaves-th slot. PVAR: a
// paged pool with a variable-length query batch (cu_q). NT: blocks read about once
// (decode-like batches), loaded non-temporally.
template <bool PAGED, bool TEMP, bool FP8, int kWaves, bool PVAR = false, bool NT = false>
__global__ __launch_bounds__(64 * kWaves) void qcentric_kernel(QcParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t ks_all[kWaves][kSub * kKStride];
  __shared__ __attribute__((aligned(16))) uint8_t vs_all[kWaves][kSub * kVStride];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  uint8_t* ks = ks_all[wave];
  uint8_t* vs = vs_all[wave];
  const int n = lane & 15;  // head column
  const int g = lane >> 4;  // 16-lane group

  // packed queries: contiguous varlen batches, or paged ones (PVAR)
  const bool varq = PAGED ? PVAR : p.cu_q != nullptr;
  long long item = blockIdx.x;
  if (PAGED && !PVAR) {
    // Workgroups are dealt round-robin over the 8 XCDs; this permutation puts the
    // Sq x splits items of one (b, hkv) on one XCD, so the blocks its query rows
    // share (the diagonal one at least) are fetched into a single L2. Groups past the
    // last multiple of 8 keep the identity order.
    const long long S = static_cast<long long>(p.Sq) * p.splits;
    const long long full = (static_cast<long long>(p.B) * p.Hkv / 8) * 8 * S;
    if (item < full) {
      const long long k = item / 8;
      item = ((item % 8) + 8 * (k / S)) * S + k % S;
    }
  }
  const int sp = static_cast<int>(item % p.splits);
  item /= p.splits;
  // the row's sequence b: its query position and count, its first key and key count
  int b, hkv;
  long long grow, qpos, sq_b, kbeg, kvlen;
  const int32_t* sel;
  if (varq) {
    grow = item % p.total_q;
    hkv = static_cast<int>(item / p.total_q);
    b = seq_search(p.cu_q, p.B, grow);
    long long qbeg;
    seq_range(p.cu_q, b, p.total_q, qbeg, sq_b);
    qpos = grow - qbeg;
    if (PAGED) {
      kbeg = 0;
      kvlen = p.seqused[b];
    } else {
      seq_range(p.cu_k, b, p.total_k, kbeg, kvlen);
    }
    sel = p.q2k + (static_cast<long long>(hkv) * p.total_q + grow) * p.topk;
  } else {
    qpos = item % p.Sq;
    item /= p.Sq;
    hkv = static_cast<int>(item % p.Hkv);
    b = static_cast<int>(item / p.Hkv);
    grow = static_cast<long long>(b) * p.Sq + qpos;
    sq_b = p.Sq;
    kbeg = static_cast<long long>(b) * p.Skv;
    kvlen = PAGED ? static_cast<long long>(p.seqused[b]) : p.Skv;
    sel = p.q2k + ((static_cast<long long>(b) * p.Hkv + hkv) * p.Sq + qpos) * p.topk;
  }
  // valid block ids: [0, nblk) (uniform or paged) or the blocks of the sequence (varlen)
  const long long nblk_b = (!PAGED && varq) ? (kvlen + kBlk - 1) / kBlk : p.nblk;

  const int head = hkv * p.qpk + n;
  const bool head_ok = n < p.qpk;

  // Q fragments: lane (n, g) holds dims 32*kq + 8*g .. +7 of head n.
  bf16x8 qf[4];
  {
    const uint16_t* qrow = p.q + (grow * p.Hq + (head_ok ? head : hkv * p.qpk)) * kD + 8 * g;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * kq);
      if (!head_ok) v = u32x4{0, 0, 0, 0};
      qf[kq] = as_bf16x8(v);
    }
  }

  long long end = kvlen;  // keys [0, end) of the sequence are visible
  if (p.causal) {
    const long long lim = qpos + kvlen - sq_b;
    if (lim + 1 < end) end = lim + 1;
  }

  const int per = (p.topk + p.splits - 1) / p.splits;
  const int t0 = sp * per;
  const int t1 = min(p.topk, t0 + per);

  // (t, u): slot t, sub-tile u; advance to the first visible one at or after it
  auto seek = [&](int& t, int& u, int& s, int& pg) {
    while (t < t1) {
      if (u < 4) {
        s = sel[t];
        bool ok = s >= 0 && s < nblk_b &&
                  static_cast<long long>(s) * kBlk + kSub * u < end;
        if (ok && PAGED) {
          pg = p.page_table[static_cast<long long>(b) * p.max_pages + s];
          ok = pg >= 0 && pg < p.num_pages;
        }
        if (ok) return;
      }
      t += kWaves;
      u = 0;
    }
  };

  // A sub-tile is 32 rows of 128 elements: 16-byte loads of 8 bf16 (8 per lane) or of
  // 16 fp8 (4 per lane, each widened to two bf16 chunks on the way to LDS).
  constexpr int kEpc = FP8 ? 16 : 8;          // elements per 16-byte load
  constexpr int kCpr = kD / kEpc;             // loads per row
  constexpr int kLpl = kSub * kCpr / 64;      // loads per lane
  constexpr int kEsz = FP8 ? 1 : 2;           // bytes per K/V element
  const char* kb = static_cast<const char*>(p.k);
  const char* vb = static_cast<const char*>(p.v);
  u32x4 kr[kLpl], vr[kLpl];
  auto load = [&](int s, int pg, int u) {
#pragma unroll
    for (int i = 0; i < kLpl; ++i) {
      const int ci = i * 64 + lane;
      const int row = ci / kCpr, c = ci % kCpr;
      long long off;  // in elements
      if (PAGED)
        off = ((static_cast<long long>(pg) * p.Hkv + hkv) * kBlk + kSub * u + row) * kD + c * kEpc;
      else  // rows past the sequence's last key re-read that key (stored as zeros)
        off = ((kbeg + min(static_cast<long long>(s) * kBlk + kSub * u + row, kvlen - 1)) * p.Hkv +
               hkv) * kD + c * kEpc;
      if (NT) {
        // blocks read about once (decode): non-temporal loads measured 6% faster on 32 x 8
        // paged queries over 65 536 keys (0.171 -> 0.161 ms, same bits); where blocks serve
        // many queries (prefill) they cost the reuse from L2 (8192 queries: 1.71 -> 2.44 ms)
        kr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kb + off * kEsz));
        vr[i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vb + off * kEsz));
      } else {
        kr[i] = *reinterpret_cast<const u32x4*>(kb + off * kEsz);
        vr[i] = *reinterpret_cast<const u32x4*>(vb + off * kEsz);
      }
    }
  };
  // keys past `end` are stored as zeros so that no value there can leak into P*V
  auto store = [&](int s, int u) {
#pragma unroll
    for (int i = 0; i < kLpl; ++i) {
      const int ci = i * 64 + lane;
      const int row = ci / kCpr, c = ci % kCpr;
      const bool ok = static_cast<long long>(s) * kBlk + kSub * u + row < end;
      const u32x4 z = {0, 0, 0, 0};
      if (FP8) {
        u32x4 kw[2], vw[2];
        fp8x16_to_bf16x16(kr[i], kw);
        fp8x16_to_bf16x16(vr[i], vw);
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          *reinterpret_cast<u32x4*>(ks + k_off(row, 2 * c + h2)) = ok ? kw[h2] : z;
          *reinterpret_cast<u32x4*>(vs + v_off(row, 2 * c + h2)) = ok ? vw[h2] : z;
        }
      } else {
        *reinterpret_cast<u32x4*>(ks + k_off(row, c)) = ok ? kr[i] : z;
        *reinterpret_cast<u32x4*>(vs + v_off(row, c)) = ok ? vr[i] : z;
      }
    }
  };

  float m_run = -INFINITY, l_run = 0.f;
  float lt_run = 0.f;  // TEMP: sum of 2^((x - m_run) / T), x the scores in log2 units
  f32x4 oacc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) oacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lq = lane & 15, rr = lq >> 2, cq = lq & 3;

  auto compute = [&](int s, int u) {
    // S^T sub-tile: 32 tokens x 16 heads, two 16-token M tiles
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int kq = 0; kq < 4; ++kq) {
        const bf16x8 a =
            as_bf16x8(*reinterpret_cast<const u32x4*>(ks + k_off(16 * mt + n, 4 * kq + g)));
        sacc[mt] = mfma16(a, qf[kq], sacc[mt]);
      }
    // lane (n, g) holds tokens 16*mt + 4*g + i of head n
    const long long jb = static_cast<long long>(s) * kBlk + kSub * u;
    float x[2][4];
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const long long j = jb + 16 * mt + 4 * g + i;
        x[mt][i] = j < end ? sacc[mt][i] * p.scale_log2 : -INFINITY;
        mx = fmaxf(mx, x[mt][i]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx);  // finite: key jb is visible
    const float alpha = fast_exp2(m_run - m_new);
    float ps = 0.f, pst = 0.f;
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (TEMP) pst += fast_exp2((x[mt][i] - m_new) * p.inv_temp);
        x[mt][i] = fast_exp2(x[mt][i] - m_new);
        ps += x[mt][i];
      }
    ps += __shfl_xor(ps, 16);
    ps += __shfl_xor(ps, 32);
    l_run = l_run * alpha + ps;
    if (TEMP) {
      pst += __shfl_xor(pst, 16);
      pst += __shfl_xor(pst, 32);
      lt_run = lt_run * fast_exp2((m_run - m_new) * p.inv_temp) + pst;
    }
    m_run = m_new;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[dt] *= alpha;
    // P^T as the B operand: k slots 8g..8g+3 = tokens 4g+i, 8g+4..8g+7 = tokens 16+4g+i
    const u32x4 pw = {pack_bf16x2(x[0][0], x[0][1]), pack_bf16x2(x[0][2], x[0][3]),
                      pack_bf16x2(x[1][0], x[1][1]), pack_bf16x2(x[1][2], x[1][3])};
    const bf16x8 pb = as_bf16x8(pw);
    // rows 4g + rr and 16 + 4g + rr, columns 16*dt + 4*cq .. +3
    const uint8_t* vrow = vs + (4 * g + rr) * kVStride + 8 * cq;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const i16x4 lo = lds_read_tr16(vrow + 32 * dt);
      const i16x4 hi = lds_read_tr16(vrow + 16 * kVStride + 32 * dt);
      oacc[dt] = mfma16(cat_tr(lo, hi), pb, oacc[dt]);
    }
  };

  int t = t0 + wave, u = 0, s = 0, pg = 0;  // this wave's slots: t0 + wave, + kWaves, ...
  seek(t, u, s, pg);
  if (t < t1) load(s, pg, u);
  while (t < t1) {
    int tn = t, un = u + 1, sn = s, pgn = pg;
    seek(tn, un, sn, pgn);
    wave_lds_sync();
    store(s, u);
    if (tn < t1) load(sn, pgn, un);
    wave_lds_sync();
    compute(s, u);
    t = tn;
    u = un;
    s = sn;
    pg = pgn;
  }

  // merge the waves' states into wave 0: wave w > 0 publishes (O, m, l[, lt]) in its V
  // tile, lane-major so that both sides access consecutive words
  if (kWaves > 1) {
    constexpr int kPub = 35;  // 32 accumulator words + m, l, lt per lane
    static_assert(kPub * 64 * 4 <= kSub * kVStride, "merge buffer exceeds the V tile");
    float* pub = reinterpret_cast<float*>(vs);
    wave_lds_sync();
    if (wave > 0) {
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i) pub[(4 * dt + i) * 64 + lane] = oacc[dt][i];
      pub[32 * 64 + lane] = m_run;
      pub[33 * 64 + lane] = l_run;
      pub[34 * 64 + lane] = lt_run;
    }
    __syncthreads();
    if (wave > 0) return;
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      const float* other = reinterpret_cast<const float*>(vs_all[w]);
      const float m1 = other[32 * 64 + lane], l1 = other[33 * 64 + lane];
      const float mm = fmaxf(m_run, m1);
      const float a0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - mm);
      const float a1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - mm);
      l_run = l_run * a0 + l1 * a1;
      if (TEMP) {
        const float b0 = m_run == -INFINITY ? 0.f : fast_exp2((m_run - mm) * p.inv_temp);
        const float b1 = m1 == -INFINITY ? 0.f : fast_exp2((m1 - mm) * p.inv_temp);
        lt_run = lt_run * b0 + other[34 * 64 + lane] * b1;
      }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          oacc[dt][i] = oacc[dt][i] * a0 + other[(4 * dt + i) * 64 + lane] * a1;
      m_run = mm;
    }
  }

  // epilogue: lane (n, g) holds dims 16*dt + 4*g + i of head n
  const bool any = l_run > 0.f;
  const float inv = any ? 1.f / l_run : 0.f;
  const float lse_v = any ? (m_run + fast_log2(l_run)) * kLn2 : -INFINITY;
  const float lset_v = any ? (m_run * p.inv_temp + fast_log2(lt_run)) * kLn2 : -INFINITY;
  if (!head_ok) return;
  if (p.splits == 1) {
    uint16_t* orow = p.o + (grow * p.Hq + head) * kD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) {
      const u32x2 w = {pack_bf16x2(oacc[dt][0] * inv, oacc[dt][1] * inv),
                       pack_bf16x2(oacc[dt][2] * inv, oacc[dt][3] * inv)};
      *reinterpret_cast<u32x2*>(orow + 16 * dt) = w;
    }
    if (g == 0) {
      const long long li = varq ? grow * p.Hq + head
                                : (static_cast<long long>(b) * p.Hq + head) * p.Sq + qpos;
      p.lse[li] = lse_v;
      if (TEMP) p.lse_t[li] = lset_v;
    }
  } else {
    // paged: rows [splits][B * Sq or total_q][Hq]
    const long long prow =
        (PAGED && PVAR) ? (static_cast<long long>(sp) * p.total_q + grow) * p.Hq + head
                        : (static_cast<long long>(sp) * p.B * p.Sq + grow) * p.Hq + head;
    float* orow = p.o_part + prow * kD + 4 * g;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) *reinterpret_cast<f32x4*>(orow + 16 * dt) = oacc[dt] * inv;
    if (g == 0) {
      p.lse_part[prow] = lse_v;
      if (TEMP) p.lse_t_part[prow] = lset_v;
    }
  }
}

template <int W, bool PAGED, bool PVAR, bool NT>
void qc_launch_tf(int tf, const QcParams& p, dim3 grid, hipStream_t stream) {
  const dim3 blk(64 * W);
  switch (tf) {  // temperature LSE (2), fp8 K/V (1)
    case 0: hipLaunchKernelGGL((qcentric_kernel<PAGED, false, false, W, PVAR, NT>), grid, blk, 0, stream, p); break;
    case 1: hipLaunchKernelGGL((qcentric_kernel<PAGED, false, true, W, PVAR, NT>), grid, blk, 0, stream, p); break;
    case 2: hipLaunchKernelGGL((qcentric_kernel<PAGED, true, false, W, PVAR, NT>), grid, blk, 0, stream, p); break;
    default: hipLaunchKernelGGL((qcentric_kernel<PAGED, true, true, W, PVAR, NT>), grid, blk, 0, stream, p); break;
  }
}

template <int W>
void qc_launch(int variant, const QcParams& p, dim3 grid, hipStream_t stream) {
  const int tf = variant & 3;
  switch (variant >> 2) {  // paged (1), packed queries (2), streamed blocks (4)
    case 0: qc_launch_tf<W, false, false, false>(tf, p, grid, stream); break;
    case 1: qc_launch_tf<W, true, false, false>(tf, p, grid, stream); break;
    case 4: qc_launch_tf<W, false, false, true>(tf, p, grid, stream); break;
    case 3: qc_launch_tf<W, true, true, false>(tf, p, grid, stream); break;
    case 5: qc_launch_tf<W, true, false, true>(tf, p, grid, stream); break;
    default: qc_launch_tf<W, true, true, true>(tf, p, grid, stream); break;
  }
}

}  // namespace

hipError_t launch_qcentric(const QcParams& p, bool paged, hipStream_t stream) {
  // packed queries (cu_q): contiguous K/V take one split
  const long long rows = p.cu_q ? p.total_q : static_cast<long long>(p.B) * p.Sq;
  const long long items = rows * p.Hkv * p.splits;
  if (p.cu_q && !paged && p.splits != 1) return hipErrorInvalidValue;
  if (items <= 0) return hipSuccess;
  if (items > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(items));
  // Two waves per row when the rows alone leave the compute units short of waves
  // (decode: the 32 x 8-query paged workload has 1024 (row, KV head) items);
  // otherwise one (large prefill, where the second wave only adds Q loads and a merge).
  const bool two = items < 8LL * device_cu_count();
  const int variant = (paged ? 4 : 0) + (paged && p.cu_q ? 8 : 0) + (p.kv_stream ? 16 : 0) +
                      (p.lse_t ? 2 : 0) + (p.kv_fp8 ? 1 : 0);
  if (two)
    qc_launch<2>(variant, p, grid, stream);
  else
    qc_launch<1>(variant, p, grid, stream);
  return hipGetLastError();
}

}  // namespace msa
