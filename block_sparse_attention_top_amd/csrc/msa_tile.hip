// Query-tile sparse attention forward for dense selections (contiguous K/V).
//
// The operation is the sparse attention of `sparse_attention_ref` on the page
// "MiniMax-AI/MSA python/fmha_sm100/cute/test_sparse_atten.py": for query
// (b, q) and KV head hkv, the qhead_per_kv query heads sharing the index row
// q2k[b][hkv][q][:] attend to the union of its valid blocks under the
// bottom-right causal limit q + Skv - Sq; natural-log LSE, (O = 0, LSE = -inf)
// for an empty key set.
//
// Organisation on gfx950. When each KV block is selected by many nearby queries
// (few blocks, causal prefill), a workgroup of 8 waves takes a tile of
// 8 * (32 / qhead_per_kv) consecutive queries of one (b, hkv) and streams the
// distinct blocks their index rows select (first-occurrence order), each block
// once, through two LDS buffers filled by direct global->LDS loads (one barrier
// per block; the tiles keep the padded row strides of the kv-centric kernel).
// Each wave owns 32 (query, head) rows -- 32 / qhead_per_kv queries -- as the
// N = 32 columns of v_mfma_f32_32x32x16_bf16 and, for every block one of
// its queries selected, computes S^T = K Q^T over the whole 128-token block
// (K fragments by ds_read_b128), an online softmax per lane column whose
// reference maximum only moves when a score exceeds it by 2^8, and
// O^T += V^T P^T (V fragments by the transposing ds_read_b64_tr_b16); rows of a
// query that did not select the block are masked. Q fragments and the O
// accumulators stay in registers for the whole tile, so nothing but O and LSE is
// written. Tiles are placed so that the XCDs serving one KV head share its K/V
// in their L2, largest (latest causal) tiles first.
#include "msa_internal.hpp"
#include "msa_lds.hpp"

#include <math.h>

namespace msa {

namespace {

constexpr int kWaves = 8;
constexpr int kMaxEnt = kTileMaxEntries;  // index entries per tile
// Block tiles in LDS use the padded row strides of the kv-centric kernel (K 272 B,
// V 320 B: conflict-free fragment reads with immediate offsets). A padded tile is
// filled as a run of 16-byte units by direct loads: unit i of the tile is chunk
// i % (stride / 16) of row i / (stride / 16); units past chunk 15 are padding and
// receive a duplicate of the row's first chunk.
constexpr int kKUnits = kKStride / 16;            // 17 units per K row
constexpr int kVUnits = kVStride / 16;            // 20 units per V row
constexpr int kKTileB = kBlk * kKStride;          // 34 KiB
constexpr int kVTileB = kBlk * kVStride;          // 40 KiB
constexpr int kBufB = kKTileB + kVTileB;          // one buffer: K tile then V tile
constexpr int kKLoads = kKTileB / 1024;           // 1 KiB per load instruction: 34
constexpr int kVLoads = kVTileB / 1024;           // 40

// s_waitcnt immediate (gfx9 encoding): vmcnt(0) lgkmcnt(0)
constexpr int kWaitAll = 0 | (7 << 4);


template <int QPK, bool TEMP>
__global__ __launch_bounds__(512, 1) void tile_kernel(TileParams p) {
  constexpr int EPW = 32 / QPK;     // queries per wave
  constexpr int T = kWaves * EPW;   // queries per tile
  static_assert(T <= kTileMaxQ, "tile too large");
  __shared__ __attribute__((aligned(1024))) uint8_t kv[2][kBufB];  // [buffer][K | V]
  __shared__ int ublk[kMaxEnt];
  __shared__ unsigned umask[kMaxEnt];
  __shared__ unsigned long long fmask[kMaxEnt / 64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // placement: workgroup id g runs on XCD g % 8
  int pair, tile;
  {
    const int g = blockIdx.x, xcd = g & 7, k = g >> 3;
    if (p.xcd_pairs) {  // pairs share XCDs: xcd % P is the pair, interleaved tiles
      const int P = p.B * p.Hkv, R = 8 / P;
      pair = xcd % P;
      tile = k * R + xcd / P;
    } else {
      pair = g / p.ntiles;
      tile = g % p.ntiles;
    }
    if (pair >= p.B * p.Hkv || tile >= p.ntiles) return;  // whole workgroup, before barriers
    tile = p.ntiles - 1 - tile;  // latest (largest causal) tiles first
  }
  const int b = pair / p.Hkv, hkv = pair % p.Hkv;
  const int q0 = tile * T;
  const int nent = T * p.topk;
  const long long off_kv = static_cast<long long>(p.Skv) - p.Sq;
  int* ent_id = reinterpret_cast<int*>(&kv[1][0]);  // union build only, before any load
  auto end_of = [&](int q) -> long long {  // keys [0, end) visible to query q
    long long e = p.Skv;
    if (p.causal && q + off_kv + 1 < e) e = q + off_kv + 1;
    return e;
  };

  // 1. valid entries of the tile's index rows
  const int32_t* sel = p.q2k + ((static_cast<long long>(b) * p.Hkv + hkv) * p.Sq + q0) * p.topk;
  for (int i = tid; i < nent; i += 512) {
    const int j = i / p.topk;
    int id = -1;
    if (q0 + j < p.Sq) {
      const int s = sel[i];
      if (s >= 0 && s < p.nblk && static_cast<long long>(s) * kBlk < end_of(q0 + j)) id = s;
    }
    ent_id[i] = id;
  }
  __syncthreads();
  // 2. distinct ids in first-occurrence order with the mask of selecting queries
  //    (one uniform pass over the entries with broadcast LDS reads, then ballot
  //    prefix counts number the first occurrences)
  constexpr int kPasses = (kMaxEnt + 511) / 512;
  bool first[kPasses];
  unsigned qm[kPasses];
  int myid[kPasses];
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    const int i = ps * 512 + tid;
    const int id = i < nent ? ent_id[i] : -1;
    bool f = id >= 0;
    unsigned m = 0;
    if (ps * 512 < nent) {  // uniform
      for (int j = 0, e = 0; j < T; ++j)
        for (int t = 0; t < p.topk; ++t, ++e)
          if (ent_id[e] == id) {
            m |= 1u << j;
            f = f && e >= i;
          }
    }
    first[ps] = f;
    qm[ps] = m;
    myid[ps] = id;
    const unsigned long long bal = __ballot(f);
    if (lane == 0) fmask[ps * kWaves + wave] = bal;
  }
  __syncthreads();
  int U = 0;
#pragma unroll
  for (int c = 0; c < kPasses * kWaves; ++c) U += __popcll(fmask[c]);
#pragma unroll
  for (int ps = 0; ps < kPasses; ++ps) {
    if (!first[ps]) continue;
    const int c = ps * kWaves + wave;
    int pos = __popcll(fmask[c] & ((1ull << lane) - 1ull));
    for (int e = 0; e < c; ++e) pos += __popcll(fmask[e]);
    ublk[pos] = myid[ps];
    umask[pos] = qm[ps];
  }

  // 3. this wave's rows: lane column n = (query e, head hi), k-half h
  const int n = lane & 31, h = lane >> 5;
  const int e = n / QPK, hi = n % QPK;
  const int qloc = wave * EPW + e;  // query index inside the tile
  const int q = q0 + qloc;
  const bool qok = q < p.Sq;
  const int head = hkv * QPK + hi;
  // Q^T fragments: lane (n, h) holds dims 16*kq + 8*h .. +7 of its row
  bf16x8 qf[8];
  {
    const uint16_t* qrow =
        p.q + ((static_cast<long long>(b) * p.Sq + (qok ? q : 0)) * p.Hq + head) * kD + 8 * h;
#pragma unroll
    for (int kq = 0; kq < 8; ++kq) {
      u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * kq);
      if (!qok) v = u32x4{0, 0, 0, 0};
      qf[kq] = as_bf16x8(v);
    }
  }
  const long long qend = qok ? end_of(q) : 0;
  const float c2 = p.scale_log2;
  const unsigned wmask = ((1u << EPW) - 1u) << (wave * EPW);  // this wave's queries
  __syncthreads();  // union list complete

  // direct loads of block u's padded K and V tiles into buffer bf: load
  // instruction i (64 units of 16 B) goes to wave i % 8
  auto issue = [&](int u, int bf) {
    const long long tok0 = static_cast<long long>(b) * p.Skv + static_cast<long long>(ublk[u]) * kBlk;
    const uint32_t kl = lds_addr(&kv[bf][0]);
    for (int i = wave; i < kKLoads + kVLoads; i += kWaves) {  // wave-uniform bounds
      const bool isk = i < kKLoads;
      const int unit = 64 * (isk ? i : i - kKLoads) + lane;
      const int upr = isk ? kKUnits : kVUnits;
      const int r = unit / upr, c = unit % upr;
      const long long row = ((tok0 + r) * p.Hkv + hkv) * kD + 8 * (c < 16 ? c : 0);
      lds_load16((isk ? p.k : p.v) + row, kl + (isk ? 0 : kKTileB) + 1024 * (isk ? i : i - kKLoads));
    }
  };

  float m_ref = -INFINITY, ls = 0.f;  // reference max (raw score units), row sum
  float lt = 0.f;  // TEMP: row sum of 2^((s - m_ref) * c2 / T)
  // the reference max moves when exceeded by 8 / max(1, 1/T) in log2 units, so that
  // neither sum's terms exceed 2^8
  const float c2t = c2 * p.inv_temp;
  const float c2m = TEMP ? c2 * fmaxf(1.f, p.inv_temp) : c2;
  f32x16 oacc[4];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};

  const int j16 = lane >> 4, lq = lane & 15, rr = lq >> 2, cq = lq & 3;
  // lane offsets inside the tiles: K fragment row n, chunk h; V transposed reads
  const int kbase0 = n * kKStride + h * 16;
  const int vbase0 = (4 * h + rr) * kVStride + 32 * (j16 & 1) + 8 * cq;
  auto compute = [&](int u, const uint8_t* ks, const uint8_t* vs) {
    const unsigned msk = umask[u];
    if (!(msk & wmask)) return;  // wave-uniform: none of this wave's queries selected it
    const long long blk0 = static_cast<long long>(ublk[u]) * kBlk;
    // visible tokens of this block for the lane's row (0 when its query did not select it)
    const bool mine = (msk >> qloc) & 1u;
    const int vis = mine ? static_cast<int>(min(qend - blk0, static_cast<long long>(kBlk))) : 0;
    const bool full = __all(vis >= kBlk);
    // opaque per block so that K fragments are re-read from LDS, not held
    int kbase = kbase0, vbase = vbase0;
    asm volatile("" : "+v"(kbase), "+v"(vbase));
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      // S^T half: tokens 64*hf + 32*mt + 8*(i/4) + 4*h + i%4 of row n
      f32x16 sacc[2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        sacc[mt] = f32x16{};
#pragma unroll
        for (int kq = 0; kq < 8; ++kq) {
          const bf16x8 a = as_bf16x8(*reinterpret_cast<const u32x4*>(
              ks + kbase + (64 * hf + 32 * mt) * kKStride + 32 * kq));
          sacc[mt] = mfma32(a, qf[kq], sacc[mt]);
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
      // the reference max moves only when exceeded by 2^8 (a row's first keys always)
      if (__any((mx - m_ref) * c2m > 8.f)) {
        const float m_new = fmaxf(m_ref, mx);
        const float alpha = m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * c2);
        ls *= alpha;
        if (TEMP) lt *= m_ref == -INFINITY ? 0.f : fast_exp2((m_ref - m_new) * c2t);
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
          ls += p0 + p1;
          if (TEMP)
            lt += fast_exp2(fmaf(sacc[mt][2 * i], c2t, nmc * p.inv_temp)) +
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
  };

  // 4. double-buffered stream of the listed blocks: block u+1 loads while u is used
  if (U > 0) {
    issue(0, 0);
    for (int u = 0; u < U; ++u) {
      __builtin_amdgcn_s_waitcnt(kWaitAll);  // own loads of block u landed, LDS reads done
      __builtin_amdgcn_s_barrier();          // everyone's loads landed; block u-1 released
      if (u + 1 < U) issue(u + 1, (u + 1) & 1);
      if (u & 1)
        compute(u, kv[1], kv[1] + kKTileB);
      else
        compute(u, kv[0], kv[0] + kKTileB);
    }
  }

  // 5. epilogue: O = O^T / sum, LSE = reference max + log(sum)
  ls += __shfl_xor(ls, 32);
  if (TEMP) lt += __shfl_xor(lt, 32);
  const bool any = ls > 0.f;
  const float inv = any ? 1.f / ls : 0.f;
  // lane (n, h) holds dims 32*dt + 8*q4 + 4*h .. +3 of row n; swapping the odd-q4
  // half of lane h=0 with the even-q4 half of lane h=1 (v_permlane32_swap) leaves
  // each lane 16 contiguous bytes: dims 32*dt + 16*pp + 8*h .. +7
  uint32_t ow[4][4][2];
#pragma unroll
  for (int dt = 0; dt < 4; ++dt)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      ow[dt][q4][0] = pack_bf16x2(oacc[dt][4 * q4 + 0] * inv, oacc[dt][4 * q4 + 1] * inv);
      ow[dt][q4][1] = pack_bf16x2(oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv);
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
  if (qok) {
    uint16_t* orow = p.o + ((static_cast<long long>(b) * p.Sq + q) * p.Hq + head) * kD;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int pp = 0; pp < 2; ++pp) {
        const u32x4 v4 = {ow[dt][2 * pp][0], ow[dt][2 * pp][1], ow[dt][2 * pp + 1][0],
                          ow[dt][2 * pp + 1][1]};
        *reinterpret_cast<u32x4*>(orow + 32 * dt + 16 * pp + 8 * h) = v4;
      }
    if (h == 0) {
      const long long li = (static_cast<long long>(b) * p.Hq + head) * p.Sq + q;
      const float mr = m_ref == -INFINITY ? 0.f : m_ref;
      p.lse[li] = any ? fmaf(mr, c2, fast_log2(ls)) * kLn2 : -INFINITY;
      if (TEMP) p.lse_t[li] = any ? fmaf(mr, c2t, fast_log2(lt)) * kLn2 : -INFINITY;
    }
  }
}

}  // namespace

bool tile_supported(int qpk, int topk) {
  return (qpk == 8 || qpk == 16) && kWaves * (32 / qpk) * topk <= kMaxEnt;
}

hipError_t launch_tile(TileParams p, hipStream_t stream) {
  if (!tile_supported(p.qpk, p.topk)) return hipErrorInvalidValue;
  const int T = kWaves * (32 / p.qpk);
  p.ntiles = (p.Sq + T - 1) / T;
  const long long pairs = static_cast<long long>(p.B) * p.Hkv;
  if (pairs <= 0 || p.ntiles <= 0) return hipSuccess;
  long long grid;
  if (pairs <= 8 && 8 % pairs == 0) {
    p.xcd_pairs = 1;
    const long long R = 8 / pairs;
    grid = 8 * ((p.ntiles + R - 1) / R);
  } else {
    p.xcd_pairs = 0;
    grid = pairs * p.ntiles;
  }
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  const dim3 g(static_cast<unsigned>(grid)), blk(512);
  const bool temp = p.lse_t != nullptr;
  if (p.qpk == 16 && temp)
    hipLaunchKernelGGL((tile_kernel<16, true>), g, blk, 0, stream, p);
  else if (p.qpk == 16)
    hipLaunchKernelGGL((tile_kernel<16, false>), g, blk, 0, stream, p);
  else if (temp)
    hipLaunchKernelGGL((tile_kernel<8, true>), g, blk, 0, stream, p);
  else
    hipLaunchKernelGGL((tile_kernel<8, false>), g, blk, 0, stream, p);
  return hipGetLastError();
}

}  // namespace msa
