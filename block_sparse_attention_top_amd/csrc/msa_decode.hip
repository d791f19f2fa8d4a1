// Paged sparse decode: split-KV over the union of the blocks that the few query
// rows of one (sequence, KV head) select, each distinct block read once.
//
// The operation is the paged sparse attention of `sparse_attention_ref` on the
// page "MiniMax-AI/MSA python/fmha_sm100/cute/test_sparse_atten.py" (pool
// addressed through page_table as in `pack_paged_kv`, keys at or past
// seqused_k masked, bottom-right causal limit q + seqused_k - Sq), organised as
// the split-KV decode of `sparse_decode_atten_func` / the decode wrapper on the
// page "MSA interface.py": each split writes a normalised fp32 partial (O, LSE)
// per (query, head), merged afterwards by log-sum-exp.
//
// Layout on gfx950. A workgroup (4 waves) takes (b, hkv, split). It first forms
// in LDS the list of distinct valid blocks selected by the Sq index rows of
// (b, hkv), in order of first occurrence, with a bit mask of the queries that
// selected each; the split takes a contiguous share of that list. The blocks
// are streamed as 32-token K/V sub-tiles through a ring of kStages LDS buffers
// filled by direct global->LDS loads (global_load_lds_dwordx4), three sub-tiles
// in flight while one is consumed, one barrier per sub-tile. Rows are stored
// unpadded (256 B) with the 16-byte chunks XOR-swizzled per row so that both
// fragment reads are free of bank conflicts. Every wave owns up to
// kMaxQPerWave queries and runs, for each of its queries whose bit is set,
// S^T = K Q^T and O^T += V^T P^T on v_mfma_f32_16x16x32_bf16 (N = the qpk
// heads) with an online softmax per lane column (and, when a temperature-scaled
// LSE is requested, a second running sum of 2^((x - m) / T) beside it).
#include "msa_internal.hpp"
#include "msa_lds.hpp"

#include <math.h>

namespace msa {

namespace {

constexpr int kSub = 32;  // tokens per sub-tile

constexpr int kRow = 256;  // bytes per K/V row in the decode tiles (no padding)

// 16-byte chunk c of row r sits at chunk position c ^ swz(r) of that row.
// K: fragment reads (ds_read_b128) take 16 consecutive rows at one chunk.
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
// V: transposed reads take 8 rows x one 32-byte chunk pair per half wave.
__device__ __forceinline__ int swz_v(int r) { return 2 * (r & 7); }

template <int QPW, bool TEMP, bool DENSE>
__global__ __launch_bounds__(256, QPW <= 2 ? 2 : 1) void paged_decode_kernel(QcParams p) {
  // ring of kStages sub-tile buffers; separate arrays keep the stage buffers
  // distinct objects for the compiler's tracking of the direct-to-LDS loads
  // (K sub-tile at offset 0, V sub-tile at kTile)
  constexpr int kTile = kSub * kRow;
  __shared__ __attribute__((aligned(1024))) uint8_t st0[2 * kTile], st1[2 * kTile];
  __shared__ __attribute__((aligned(1024))) uint8_t st2[2 * kTile], st3[2 * kTile];
  __shared__ int ent_id[kDecMaxEntries];
  __shared__ int ublk[kDecMaxEntries];
  __shared__ int upage[kDecMaxEntries];
  __shared__ unsigned umask[kDecMaxEntries];
  __shared__ unsigned long long fmask[4 * kDecPasses];

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  long long item = blockIdx.x;
  int sp, hkv, b;
  int4 work = {0, 0, 0, 0};  // DENSE: (b, chunk, first page, pages)
  if (DENSE) {
    hkv = static_cast<int>(item % p.Hkv);
    const long long w = item / p.Hkv;
    if (w >= *p.dec_work_count) return;  // padding past the schedule's items
    work = p.dec_items[w];
    b = work.x;
    sp = work.y;
  } else {
    sp = static_cast<int>(item % p.splits);
    item /= p.splits;
    hkv = static_cast<int>(item % p.Hkv);
    b = static_cast<int>(item / p.Hkv);
  }
  long long kvlen = p.seqused[b];
  if (DENSE) kvlen = kvlen < 0 ? 0 : min(kvlen, static_cast<long long>(p.max_pages) * kBlk);
  const int nent = DENSE ? 0 : p.Sq * p.topk;
  const int32_t* sel =
      DENSE ? nullptr : p.q2k + (static_cast<long long>(b) * p.Hkv + hkv) * p.Sq * p.topk;

  // visible key range [0, end_q) of query q
  auto end_of = [&](int q) -> long long {
    long long e = kvlen;
    if (p.causal) {
      const long long lim = q + kvlen - p.Sq;
      if (lim + 1 < e) e = lim + 1;
    }
    return e;
  };

  // per-wave query state; the Q fragments are loaded first so that they have
  // landed before the streaming loop (whose waits then cover only K/V loads)
  const int n = lane & 15, g = lane >> 4;
  const int head = hkv * p.qpk + n;
  const bool head_ok = n < p.qpk;
  bf16x8 qf[QPW][4];
  float m_run[QPW], l_run[QPW];
  float lt_run[QPW];  // TEMP: sum of 2^((x - m_run) / T), x the scores in log2 units
  f32x4 oacc[QPW][8];
  long long qend[QPW];
#pragma unroll
  for (int k = 0; k < QPW; ++k) {
    const int q = wave + 4 * k;
    const int qq = q < p.Sq ? q : 0;
    qend[k] = q < p.Sq ? end_of(q) : 0;
    const uint16_t* qrow = p.q + ((static_cast<long long>(b) * p.Sq + qq) * p.Hq +
                                  (head_ok ? head : hkv * p.qpk)) * kD + 8 * g;
#pragma unroll
    for (int kq = 0; kq < 4; ++kq) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 32 * kq);
      if (!head_ok) v = u32x4{0, 0, 0, 0};
      qf[k][kq] = as_bf16x8(v);
    }
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
    lt_run[k] = 0.f;
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) oacc[k][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  int U = 0;
  if (DENSE) {
    // the chunk's pages in order, selected by every query; a page id outside the
    // pool is read as page 0 (in bounds) and selected by no query
    U = work.w;
    const unsigned all = p.Sq >= 32 ? 0xFFFFFFFFu : ((1u << p.Sq) - 1u);
    for (int u = tid; u < U; u += 256) {
      const int s = work.z + u;
      const int pg = p.page_table[static_cast<long long>(b) * p.max_pages + s];
      const bool ok = pg >= 0 && pg < p.num_pages;
      ublk[u] = s;
      upage[u] = ok ? pg : 0;
      umask[u] = ok ? all : 0u;
    }
    __syncthreads();
  } else {
  // 1. valid entries: id in range, page in range, block starts before the row's end
  for (int i = tid; i < nent; i += 256) {
    const int q = i / p.topk;
    const int s = sel[i];
    int id = -1;
    if (s >= 0 && s < p.nblk && static_cast<long long>(s) * kBlk < end_of(q)) {
      const int pg = p.page_table[static_cast<long long>(b) * p.max_pages + s];
      if (pg >= 0 && pg < p.num_pages) id = s;
    }
    ent_id[i] = id;
  }
  __syncthreads();
  // 2. for entry i: whether it is the first occurrence of its id, and the mask of
  //    the queries that select that id (one uniform pass, broadcast LDS reads);
  //    the first occurrences are then numbered by ballot prefix counts
  bool first[kDecPasses];
  unsigned qmask[kDecPasses];
#pragma unroll
  for (int ps = 0; ps < kDecPasses; ++ps) {
    const int i = ps * 256 + tid;
    if (ps * 256 >= nent) {  // uniform
      first[ps] = false;
      qmask[ps] = 0;
      if (lane == 0) fmask[ps * 4 + wave] = 0ull;
      continue;
    }
    const int id = i < nent ? ent_id[i] : -1;
    bool f = id >= 0;
    unsigned m = 0;
    for (int q = 0, j = 0; q < p.Sq; ++q)
      for (int t = 0; t < p.topk; ++t, ++j) {
        if (ent_id[j] == id) {
          m |= 1u << q;
          f = f && j >= i;
        }
      }
    first[ps] = f;
    qmask[ps] = m;
    const unsigned long long bal = __ballot(f);
    if (lane == 0) fmask[ps * 4 + wave] = bal;
  }
  __syncthreads();
#pragma unroll
  for (int c = 0; c < 4 * kDecPasses; ++c) U += __popcll(fmask[c]);
#pragma unroll
  for (int ps = 0; ps < kDecPasses; ++ps) {
    if (!first[ps]) continue;
    const int c = ps * 4 + wave;
    int pos = __popcll(fmask[c] & ((1ull << lane) - 1ull));
    for (int e = 0; e < c; ++e) pos += __popcll(fmask[e]);
    const int id = ent_id[ps * 256 + tid];
    ublk[pos] = id;
    upage[pos] = p.page_table[static_cast<long long>(b) * p.max_pages + id];
    umask[pos] = qmask[ps];
  }
  __syncthreads();
  }  // sparse union
  const int u0 = DENSE ? 0 : static_cast<int>(static_cast<long long>(U) * sp / p.splits);
  const int u1 = DENSE ? U : static_cast<int>(static_cast<long long>(U) * (sp + 1) / p.splits);

  // Sub-tile stream: (u, sub) for u in [u0, u1) and sub < 4 while some query
  // sees it. A stage past the end re-reads the last issued sub-tile (in bounds,
  // cache-hot) so that every phase issues the same number of loads.
  const long long rowend = end_of(p.Sq - 1);  // the last query sees the most keys
  auto visible = [&](int u, int sub) {
    return static_cast<long long>(ublk[u]) * kBlk + kSub * sub < rowend;
  };
  auto advance = [&](int& u, int& sub) {
    ++sub;
    while (u < u1 && (sub >= 4 || !visible(u, sub))) {
      ++u;
      sub = 0;
    }
  };
  // Direct loads of one sub-tile: each wave writes 4-row groups 2w and 2w+1 of K
  // and of V; lane l fills row 4*grp + l/16, chunk position l%16. Rows at or
  // past the sequence end are read from its last row instead (finite data whose
  // probabilities are exactly zero), so no masked value reaches the products.
  const int lrow = lane >> 4, lpos = lane & 15;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int u, int sub, uint8_t* kd, uint8_t* vd) {
    const long long jb = static_cast<long long>(ublk[u]) * kBlk + kSub * sub;
    const long long base = (static_cast<long long>(upage[u]) * p.Hkv + hkv) * kBlk + kSub * sub;
    const long long last = rowend - 1 - jb;  // >= 0 for a visible sub-tile
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int r = 4 * (2 * wave + j) + lrow;
      const long long rs = r < last ? r : last;
      const uint16_t* ksrc = static_cast<const uint16_t*>(p.k) + (base + rs) * kD + 8 * (lpos ^ swz_k(r));
      const uint16_t* vsrc = static_cast<const uint16_t*>(p.v) + (base + rs) * kD + 8 * (lpos ^ swz_v(r));
      lds_load16_nt(ksrc, lds_addr(kd) + 4 * (2 * wave_u + j) * kRow);
      lds_load16_nt(vsrc, lds_addr(vd) + 4 * (2 * wave_u + j) * kRow);
    }
  };

  const int rr = (lane & 15) >> 2, cq = lane & 3;
  auto compute = [&](int u, int sub, const uint8_t* ks, const uint8_t* vs) {
    const unsigned msk = umask[u];
    const long long jb = static_cast<long long>(ublk[u]) * kBlk + kSub * sub;
#pragma unroll
    for (int k = 0; k < QPW; ++k) {
      const int q = wave + 4 * k;
      if (q >= p.Sq || !((msk >> q) & 1u) || jb >= qend[k]) continue;  // wave-uniform
      f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int kq = 0; kq < 4; ++kq) {
          const int r = 16 * mt + n;
          const bf16x8 a = as_bf16x8(
              *reinterpret_cast<const u32x4*>(ks + r * kRow + 16 * ((4 * kq + g) ^ swz_k(r))));
          sacc[mt] = mfma16(a, qf[k][kq], sacc[mt]);
        }
      float x[2][4];
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const long long j = jb + 16 * mt + 4 * g + i;
          x[mt][i] = j < qend[k] ? sacc[mt][i] * p.scale_log2 : -INFINITY;
          mx = fmaxf(mx, x[mt][i]);
        }
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[k], mx);  // finite: key jb is visible to q
      const float alpha = fast_exp2(m_run[k] - m_new);
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
      l_run[k] = l_run[k] * alpha + ps;
      if (TEMP) {
        pst += __shfl_xor(pst, 16);
        pst += __shfl_xor(pst, 32);
        lt_run[k] = lt_run[k] * fast_exp2((m_run[k] - m_new) * p.inv_temp) + pst;
      }
      m_run[k] = m_new;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) oacc[k][dt] *= alpha;
      // P^T as the B operand: k slots 8g..8g+3 = tokens 4g+i, 8g+4..8g+7 = tokens 16+4g+i
      const u32x4 pw = {pack_bf16x2(x[0][0], x[0][1]), pack_bf16x2(x[0][2], x[0][3]),
                        pack_bf16x2(x[1][0], x[1][1]), pack_bf16x2(x[1][2], x[1][3])};
      const bf16x8 pb = as_bf16x8(pw);
      // rows 4g + rr and 16 + 4g + rr (same swizzle), columns 16*dt + 4*cq .. +3
      const int r = 4 * g + rr;
      const uint8_t* vrow = vs + r * kRow + 8 * cq;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const int off = 32 * (dt ^ (r & 7));
        const i16x4 lo = lds_read_tr16(vrow + off);
        const i16x4 hi = lds_read_tr16(vrow + 16 * kRow + off);
        oacc[k][dt] = mfma16(cat_tr(lo, hi), pb, oacc[k][dt]);
      }
    }
  };

  // Ring of four stages: while stage t is consumed, stages t+1 and t+2 are in
  // flight and stage t+3 is issued into the buffer that t-1 used (free once every
  // wave has passed this phase's barrier). Each wave issues 4 loads per stage, so
  // "own loads of stage t landed" is vmcnt <= 8; the barrier then makes every
  // wave's share visible. The phases are unrolled so each names its buffers.
  int ua = u0, sa = -1;
  advance(ua, sa);  // first visible sub-tile
  if (ua < u1) {
    int t_u[4], t_s[4];  // the sub-tile held by each buffer
    t_u[0] = ua; t_s[0] = sa;
    int nu = ua, ns = sa;
    int lu = ua, ls = sa;  // last valid sub-tile issued (the re-read target)
#define MSA_NEXT(bufi)                                   \
    do {                                                 \
      if (nu < u1) advance(nu, ns);                      \
      if (nu < u1) { lu = nu; ls = ns; }                 \
      t_u[bufi] = nu; t_s[bufi] = ns;                    \
    } while (0)
    issue(ua, sa, st0, st0 + kTile);
    MSA_NEXT(1);
    issue(lu, ls, st1, st1 + kTile);
    MSA_NEXT(2);
    issue(lu, ls, st2, st2 + kTile);
#define MSA_PHASE(cur, kc, vc, nxt, kn, vn)                                      \
    {                                                                            \
      __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(8));                           \
      __builtin_amdgcn_s_barrier();                                              \
      MSA_NEXT(nxt);                                                             \
      issue(lu, ls, kn, vn);                                                     \
      compute(t_u[cur], t_s[cur], kc, vc);                                       \
      if (t_u[(cur + 1) & 3] >= u1) break;                                       \
    }
    while (true) {
      MSA_PHASE(0, st0, st0 + kTile, 3, st3, st3 + kTile)
      MSA_PHASE(1, st1, st1 + kTile, 0, st0, st0 + kTile)
      MSA_PHASE(2, st2, st2 + kTile, 1, st1, st1 + kTile)
      MSA_PHASE(3, st3, st3 + kTile, 2, st2, st2 + kTile)
    }
#undef MSA_PHASE
#undef MSA_NEXT
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm0(0));  // no load outlives the loop
  }

  // 4. epilogue: lane (n, g) holds dims 16*dt + 4*g + i of head n
  if (!head_ok) return;
#pragma unroll
  for (int k = 0; k < QPW; ++k) {
    const int q = wave + 4 * k;
    if (q >= p.Sq) continue;
    const bool any = l_run[k] > 0.f;
    const float inv = any ? 1.f / l_run[k] : 0.f;
    const float lse_v = any ? (m_run[k] + fast_log2(l_run[k])) * kLn2 : -INFINITY;
    const float lset_v =
        any ? (m_run[k] * p.inv_temp + fast_log2(lt_run[k])) * kLn2 : -INFINITY;
    const long long grow = static_cast<long long>(b) * p.Sq + q;
    const int count = DENSE ? p.dec_counts[b] : p.splits;
    if (count == 1) {
      uint16_t* orow = p.o + (grow * p.Hq + head) * kD + 4 * g;
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const u32x2 w = {pack_bf16x2(oacc[k][dt][0] * inv, oacc[k][dt][1] * inv),
                         pack_bf16x2(oacc[k][dt][2] * inv, oacc[k][dt][3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 16 * dt) = w;
      }
      if (g == 0) {
        const long long li = (static_cast<long long>(b) * p.Hq + head) * p.Sq + q;
        p.lse[li] = lse_v;
        if (TEMP) p.lse_t[li] = lset_v;
      }
    } else {
      // a split that saw no key of this query leaves its O partial unwritten:
      // the split combine reads O only where the partial LSE is finite
      const long long prow =
          DENSE ? (static_cast<long long>(p.dec_o_indptr[b]) + static_cast<long long>(q) * count + sp) *
                          p.Hq + head
                : (static_cast<long long>(sp) * p.B * p.Sq + grow) * p.Hq + head;
      if (any) {
        float* orow = p.o_part + prow * kD + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
          *reinterpret_cast<f32x4*>(orow + 16 * dt) = oacc[k][dt] * inv;
      }
      if (g == 0) {
        p.lse_part[prow] = lse_v;
        if (TEMP) p.lse_t_part[prow] = lset_v;
      }
    }
  }
}

template <int QPW, bool DENSE>
void decode_launch(const QcParams& p, dim3 grid, hipStream_t stream) {
  if (p.lse_t)
    hipLaunchKernelGGL((paged_decode_kernel<QPW, true, DENSE>), grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((paged_decode_kernel<QPW, false, DENSE>), grid, dim3(256), 0, stream, p);
}

template <bool DENSE>
hipError_t decode_dispatch(const QcParams& p, dim3 grid, hipStream_t stream) {
  switch ((p.Sq + 3) / 4) {
    case 1: decode_launch<1, DENSE>(p, grid, stream); break;
    case 2: decode_launch<2, DENSE>(p, grid, stream); break;
    case 3: decode_launch<3, DENSE>(p, grid, stream); break;
    case 4: decode_launch<4, DENSE>(p, grid, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool paged_decode_supported(int Sq, int topk) {
  return Sq >= 1 && Sq <= 4 * kMaxQPerWave && Sq * topk <= kDecMaxEntries;
}

hipError_t launch_paged_decode(const QcParams& p, hipStream_t stream) {
  const long long items = static_cast<long long>(p.B) * p.Hkv * p.splits;
  if (items <= 0) return hipSuccess;
  if (items > 0x7FFFFFFFLL || !paged_decode_supported(p.Sq, p.topk)) return hipErrorInvalidValue;
  return decode_dispatch<false>(p, dim3(static_cast<unsigned>(items)), stream);
}

hipError_t launch_dense_decode_grouped(const QcParams& p, int padded_work, hipStream_t stream) {
  const long long items = static_cast<long long>(padded_work) * p.Hkv;
  if (items <= 0) return hipSuccess;
  if (items > 0x7FFFFFFFLL || p.Sq < 1 || p.Sq > 4 * kMaxQPerWave) return hipErrorInvalidValue;
  return decode_dispatch<true>(p, dim3(static_cast<unsigned>(items)), stream);
}

}  // namespace msa
