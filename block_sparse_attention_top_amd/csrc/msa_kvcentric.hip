// kv-centric sparse attention forward: per-KV-block partials driven by the
// k2q CSR, merged afterwards by the slot combine.
//
// This follows the structure of the pages' sparse forward: `sparse_atten_func`
// on the page "MSA interface.py" consumes the kv-block -> query CSR from
// `build_k2q_csr`, computes for each (KV block, queries that selected it) a
// block-local softmax and a normalised partial output plus its LSE, and merges
// the partials of each query by log-sum-exp in a separate `combine` step (its
// split-K semantics are the `o_partial_dtype` branch of `sparse_attention_ref`
// on the page "test_sparse_atten.py"). Partials are bf16 (the pages' default
// partial dtype) with fp32 LSE, indexed by the slot t of the index row.
//
// Layout on gfx950: a work item is (KV head, CSR row = (b, block), a chunk of
// up to `chunk_entries` CSR entries). The workgroup (4 waves) stages the
// block's K and V tiles (128 x 128 bf16 each) in LDS once; each wave then
// takes 32 gathered (query, head) rows at a time as the N = 32 columns of
// v_mfma_f32_32x32x16_bf16: S^T = K Q^T with K fragments from LDS and Q rows
// loaded straight from HBM, a block-local softmax per lane column, and
// O^T = V^T P^T with V fragments from the transposing ds_read_b64_tr_b16.
#include "msa_internal.hpp"

#include <math.h>

namespace msa {

namespace {

template <int QPK>
__global__ __launch_bounds__(256) void kvcentric_kernel(KvParams p) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * kBlk * 256];
  uint8_t* ks = lds;
  uint8_t* vs = lds + kBlk * 256;

  const int nitems = p.Hkv * p.nrows;
  const int total = p.chunk_ptr[nitems];
  const int w = blockIdx.x;
  if (w >= total) return;
  // the (hkv, row) whose chunk range holds w
  int lo = 0, hi = nitems;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (p.chunk_ptr[mid] <= w) lo = mid; else hi = mid;
  }
  const int hkv = lo / p.nrows, r = lo % p.nrows;
  const int* rp = p.row_ptr + static_cast<long long>(hkv) * (p.nrows + 1);
  const int e0 = rp[r] + (w - p.chunk_ptr[lo]) * p.chunk_entries;
  const int e1 = min(e0 + p.chunk_entries, rp[r + 1]);
  const int b = r / p.nblk, s = r % p.nblk;

  // stage K and V of block s (128 tokens x 256 B each)
  {
    const int tid = threadIdx.x;
    const long long tok0 = static_cast<long long>(b) * p.Skv + static_cast<long long>(s) * kBlk;
    u32x4 kr[8], vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ci = i * 256 + tid;
      const int row = ci >> 4, c = ci & 15;
      const long long off = ((tok0 + row) * p.Hkv + hkv) * kD + c * 8;
      kr[i] = *reinterpret_cast<const u32x4*>(p.k + off);
      vr[i] = *reinterpret_cast<const u32x4*>(p.v + off);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ci = i * 256 + tid;
      const int row = ci >> 4, c = ci & 15;
      *reinterpret_cast<u32x4*>(ks + lds_chunk_off(row, c)) = kr[i];
      *reinterpret_cast<u32x4*>(vs + lds_chunk_off(row, c)) = vr[i];
    }
  }
  __syncthreads();

  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int n = lane & 31;   // row column of the 32x32 MFMA
  const int h = lane >> 5;   // k-half
  constexpr int EPW = 32 / QPK;  // CSR entries per wave step
  const int ent = n / QPK, head_i = n % QPK;
  const int head = hkv * QPK + head_i;
  const long long cap = p.cap;
  const int j16 = lane >> 4, lq = lane & 15, rr = lq >> 2, cq = lq & 3;
  const long long lim_off = static_cast<long long>(p.Skv) - p.Sq;
  const long long blk0 = static_cast<long long>(s) * kBlk;

  for (int eb = e0 + wave * EPW; eb < e1; eb += 4 * EPW) {
    const int e = eb + ent;
    const bool ok = e < e1;
    int gq = 0, t = 0;
    if (ok) {
      gq = p.q_idx[hkv * cap + e];
      t = p.slot[hkv * cap + e];
    }
    const int qpos = gq % p.Sq;
    bf16x8 qf[8];
    {
      const uint16_t* qrow = p.q + (static_cast<long long>(gq) * p.Hq + head) * kD + 8 * h;
#pragma unroll
      for (int kq = 0; kq < 8; ++kq) {
        u32x4 v = *reinterpret_cast<const u32x4*>(qrow + 16 * kq);
        if (!ok) v = u32x4{0, 0, 0, 0};
        qf[kq] = as_bf16x8(v);
      }
    }
    // S^T: 128 tokens (4 M tiles of 32) x 32 rows
    f32x16 sacc[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      sacc[mt] = f32x16{};
#pragma unroll
      for (int kq = 0; kq < 8; ++kq) {
        const bf16x8 a =
            as_bf16x8(*reinterpret_cast<const u32x4*>(ks + lds_chunk_off(32 * mt + n, 2 * kq + h)));
        sacc[mt] = mfma32(a, qf[kq], sacc[mt]);
      }
    }
    // lane (n, h) holds tokens 32*mt + 8*(i/4) + 4*h + i%4 of row n
    const long long lim = p.causal ? qpos + lim_off : (1LL << 62);
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const long long j = blk0 + 32 * mt + 8 * (i >> 2) + 4 * h + (i & 3);
        const float x = (ok && j <= lim) ? sacc[mt][i] * p.scale_log2 : -INFINITY;
        sacc[mt][i] = x;
        mx = fmaxf(mx, x);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mref = mx == -INFINITY ? 0.f : mx;
    float ps = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pv = fast_exp2(sacc[mt][i] - mref);
        sacc[mt][i] = pv;
        ps += pv;
      }
    ps += __shfl_xor(ps, 32);

    f32x16 oacc[4];
#pragma unroll
    for (int dt = 0; dt < 4; ++dt) oacc[dt] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < 8; ++kk) {
      const int mt = kk >> 1, i0 = 8 * (kk & 1);
      const u32x4 pw = {pack_bf16x2(sacc[mt][i0 + 0], sacc[mt][i0 + 1]),
                        pack_bf16x2(sacc[mt][i0 + 2], sacc[mt][i0 + 3]),
                        pack_bf16x2(sacc[mt][i0 + 4], sacc[mt][i0 + 5]),
                        pack_bf16x2(sacc[mt][i0 + 6], sacc[mt][i0 + 7])};
      const bf16x8 pb = as_bf16x8(pw);
      const int r1 = 16 * kk + 4 * h + rr, r2 = r1 + 8;
#pragma unroll
      for (int dt = 0; dt < 4; ++dt) {
        const int c = 4 * dt + 2 * (j16 & 1) + (cq >> 1);
        const int half = (cq & 1) * 8;
        const i16x4 lo4 = lds_read_tr16(vs + lds_chunk_off(r1, c) + half);
        const i16x4 hi4 = lds_read_tr16(vs + lds_chunk_off(r2, c) + half);
        oacc[dt] = mfma32(cat_tr(lo4, hi4), pb, oacc[dt]);
      }
    }
    if (!ok) continue;
    // lane (n, h) holds dims 32*dt + 8*(i/4) + 4*h + i%4 of row n
    const float inv = ps > 0.f ? 1.f / ps : 0.f;
    const long long prow = (static_cast<long long>(gq) * p.topk + t) * p.Hq + head;
    uint16_t* orow = p.o_part + prow * kD + 4 * h;
#pragma unroll
    for (int dt = 0; dt < 4; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const u32x2 v2 = {pack_bf16x2(oacc[dt][4 * q4 + 0] * inv, oacc[dt][4 * q4 + 1] * inv),
                          pack_bf16x2(oacc[dt][4 * q4 + 2] * inv, oacc[dt][4 * q4 + 3] * inv)};
        *reinterpret_cast<u32x2*>(orow + 32 * dt + 8 * q4) = v2;
      }
    if (h == 0) p.lse_part[prow] = ps > 0.f ? (mx + fast_log2(ps)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_kvcentric(const KvParams& p, int grid, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  switch (p.qpk) {
    case 1: hipLaunchKernelGGL(kvcentric_kernel<1>, dim3(grid), dim3(256), 0, stream, p); break;
    case 2: hipLaunchKernelGGL(kvcentric_kernel<2>, dim3(grid), dim3(256), 0, stream, p); break;
    case 4: hipLaunchKernelGGL(kvcentric_kernel<4>, dim3(grid), dim3(256), 0, stream, p); break;
    case 8: hipLaunchKernelGGL(kvcentric_kernel<8>, dim3(grid), dim3(256), 0, stream, p); break;
    case 16: hipLaunchKernelGGL(kvcentric_kernel<16>, dim3(grid), dim3(256), 0, stream, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace msa
