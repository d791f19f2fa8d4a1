// Log-sum-exp merge of partial attention outputs.
//
// For query row (b, q) and head h with partials (O_s, L_s) over disjoint key
// sets: L = log sum_s exp(L_s) and O = sum_s exp(L_s - L) O_s; a partial with
// L_s = -inf (no visible key) carries no weight, and when every partial is
// empty the result is (O = 0, LSE = -inf). This is the `combine` step of
// `sparse_atten_func` (page "MSA interface.py") and the split-K accumulation
// of `sparse_attention_ref` (page "test_sparse_atten.py").
//
// 16 threads per (row, head), one per 8-dim chunk: 16-byte partial loads,
// fp32 accumulation, one 16-byte bf16 store; the first chunk writes the LSE.
#include "msa_internal.hpp"

#include <math.h>

namespace msa {

namespace {

// slot partials: unnormalised U_t (bf16) laid out per (query, slot, KV head) as
// [16 dim chunks][qpk heads][8 dims], with (LSE_t, M_t) [B*Sq][topk][Hq], so
// that O = sum_t e^(M_t - L) U_t; slot t of (b, q, h) exists iff
// q2k[b][h/qpk][q][t] is a valid block id. A block of 256 threads merges 16
// consecutive (query, head) rows. Weights: thread (row, t % 16) takes slots t
// and t + 16, the row's max and sum of e^(LSE_t) come from shuffles inside its
// 16-lane group, and e^(M_t - L) goes to LDS. Sums: thread = dim chunk * 16 +
// row streams its 16-byte chunk of every weighted partial (all loads issued
// together), so a wave reads whole runs of heads.
__global__ __launch_bounds__(256) void combine_slots_kernel(
    const uint16_t* __restrict__ o_part, const float2* __restrict__ lse_part,
    const int32_t* __restrict__ q2k, int B, int Sq, int Hq, int Hkv, int topk, int nblk,
    const int2* __restrict__ q_rows, uint16_t* __restrict__ o, float* __restrict__ lse,
    const float* __restrict__ lse_t_part, float* __restrict__ lse_t) {
  __shared__ float wts[16][kMaxTopk];
  __shared__ float row_lse[16];
  __shared__ float row_lse_t[16];
  const long long rows = static_cast<long long>(B) * Sq * Hq;  // varlen: B = 1, Sq = total_q
  const long long rh0 = static_cast<long long>(blockIdx.x) * 16;
  const int tid = threadIdx.x;
  const int qpk = Hq / Hkv;
  {
    const int rl = tid >> 4, t0 = tid & 15;
    const long long rh = rh0 + rl;
    float l[2] = {-INFINITY, -INFINITY}, mr[2] = {0.f, 0.f};
    float lt[2] = {-INFINITY, -INFINITY};  // temperature-scaled block LSEs
    if (rh < rows) {
      const long long gq = rh / Hq;
      const int head = static_cast<int>(rh % Hq);
      const int b = static_cast<int>(gq / Sq), qpos = static_cast<int>(gq % Sq);
      // varlen (q_rows set): q2k [Hkv][total_q][topk], valid ids below the sequence's block count
      const int32_t* row = q2k + ((static_cast<long long>(b) * Hkv + head / qpk) * Sq + qpos) * topk;
      const int nb = q_rows ? q_rows[gq].y : nblk;
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const int t = t0 + 16 * k;
        if (t < topk) {
          const int sblk = row[t];
          if (sblk >= 0 && sblk < nb) {
            const float2 lm = lse_part[(gq * topk + t) * Hq + head];
            l[k] = lm.x;
            mr[k] = lm.y;
            if (lse_t_part) lt[k] = lse_t_part[(gq * topk + t) * Hq + head];
          }
        }
      }
    }
    float m = fmaxf(l[0], l[1]);
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) m = fmaxf(m, __shfl_xor(m, d, 16));
    float sum = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int k = 0; k < 2; ++k)
        if (l[k] != -INFINITY) sum += fast_exp2((l[k] - m) * kLog2e);
    }
#pragma unroll
    for (int d = 8; d >= 1; d >>= 1) sum += __shfl_xor(sum, d, 16);
    const float L = m == -INFINITY ? -INFINITY : fmaf(fast_log2(sum), kLn2, m);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int t = t0 + 16 * k;
      if (t < topk)
        wts[rl][t] = (l[k] == -INFINITY || L == -INFINITY) ? 0.f : fast_exp2((mr[k] - L) * kLog2e);
    }
    if (t0 == 0) row_lse[rl] = L;
    if (lse_t_part) {  // the same log-sum-exp over the temperature-scaled block LSEs
      float mt = fmaxf(lt[0], lt[1]);
#pragma unroll
      for (int d = 8; d >= 1; d >>= 1) mt = fmaxf(mt, __shfl_xor(mt, d, 16));
      float st = 0.f;
      if (mt != -INFINITY) {
#pragma unroll
        for (int k = 0; k < 2; ++k)
          if (lt[k] != -INFINITY) st += fast_exp2((lt[k] - mt) * kLog2e);
      }
#pragma unroll
      for (int d = 8; d >= 1; d >>= 1) st += __shfl_xor(st, d, 16);
      if (t0 == 0) row_lse_t[rl] = mt == -INFINITY ? -INFINITY : fmaf(fast_log2(st), kLn2, mt);
    }
  }
  __syncthreads();
  const int rl = tid & 15, dc = tid >> 4;
  const long long rh = rh0 + rl;
  if (rh >= rows) return;
  const long long gq = rh / Hq;
  const int head = static_cast<int>(rh % Hq);
  const int hkv = head / qpk, head_i = head % qpk;
  const uint16_t* base = o_part + (dc * qpk + head_i) * 8;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  // eight slots' loads in flight per thread keeps the kernel at ~64 VGPRs, so more
  // blocks per CU overlap their weight phase with other blocks' loads
  constexpr int kBatch = 8;
  for (int t0 = 0; t0 < topk; t0 += kBatch) {
    u32x4 raw[kBatch];
    float wgt[kBatch];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const int t = t0 + k;
      wgt[k] = t < topk ? wts[rl][t] : 0.f;
      const long long blk = (gq * topk + t) * Hkv + hkv;
      raw[k] = wgt[k] > 0.f ? __builtin_nontemporal_load(
                                  reinterpret_cast<const u32x4*>(base + blk * (qpk * kD)))
                            : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int k = 0; k < kBatch; ++k)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[2 * i] += wgt[k] * __uint_as_float(raw[k][i] << 16);
        acc[2 * i + 1] += wgt[k] * __uint_as_float(raw[k][i] & 0xFFFF0000u);
      }
  }
  const u32x4 out = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  *reinterpret_cast<u32x4*>(o + rh * kD + 8 * dc) = out;
  if (dc == 0) {
    long long li = rh;  // varlen: [total_q][Hq]
    if (!q_rows) {
      const int b = static_cast<int>(gq / Sq), qpos = static_cast<int>(gq % Sq);
      li = (static_cast<long long>(b) * Hq + head) * Sq + qpos;
    }
    lse[li] = row_lse[rl];
    if (lse_t_part) lse_t[li] = row_lse_t[rl];
  }
}

// split partials [splits][B*Sq][Hq][D] (fp32) and [splits][B*Sq][Hq]
__global__ __launch_bounds__(256) void combine_splits_kernel(
    const float* __restrict__ o_part, const float* __restrict__ lse_part, int B, int Sq, int Hq,
    int splits, uint16_t* __restrict__ o, float* __restrict__ lse,
    const float* __restrict__ lse_t_part, float* __restrict__ lse_t) {
  const long long idx = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
  const long long rows = static_cast<long long>(B) * Sq * Hq;
  if (idx >= rows * 16) return;
  const int dc = static_cast<int>(idx & 15);
  const long long rh = idx >> 4;  // (gq, head)
  const int head = static_cast<int>(rh % Hq);
  const long long gq = rh / Hq;
  float m = -INFINITY;
  for (int sp = 0; sp < splits; ++sp) m = fmaxf(m, lse_part[sp * rows + rh]);
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float L = -INFINITY;
  if (m != -INFINITY) {
    float sum = 0.f;
    for (int sp = 0; sp < splits; ++sp) sum += expf(lse_part[sp * rows + rh] - m);
    L = m + logf(sum);
    for (int sp = 0; sp < splits; ++sp) {
      const float l = lse_part[sp * rows + rh];
      if (l == -INFINITY) continue;
      const float wgt = expf(l - L);
      const float* src = o_part + (sp * rows + rh) * kD + 8 * dc;
      const f32x4 a = *reinterpret_cast<const f32x4*>(src);
      const f32x4 c = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] += wgt * a[i];
        acc[4 + i] += wgt * c[i];
      }
    }
  }
  const u32x4 out = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
  *reinterpret_cast<u32x4*>(o + rh * kD + 8 * dc) = out;
  if (dc == 0) {
    const int b = static_cast<int>(gq / Sq), qpos = static_cast<int>(gq % Sq);
    const long long li = (static_cast<long long>(b) * Hq + head) * Sq + qpos;
    lse[li] = L;
    if (lse_t_part) {  // log-sum-exp of the splits' temperature-scaled LSEs
      float mt = -INFINITY;
      for (int sp = 0; sp < splits; ++sp) mt = fmaxf(mt, lse_t_part[sp * rows + rh]);
      float st = 0.f;
      if (mt != -INFINITY)
        for (int sp = 0; sp < splits; ++sp) st += expf(lse_t_part[sp * rows + rh] - mt);
      lse_t[li] = mt == -INFINITY ? -INFINITY : mt + logf(st);
    }
  }
}

}  // namespace

hipError_t launch_combine_slots(const uint16_t* o_part, const float2* lse_part, const int32_t* q2k,
                                int B, int Sq, int Hq, int Hkv, int topk, int nblk, uint16_t* o,
                                float* lse, hipStream_t stream, const CombineVarlen* v,
                                const float* lse_t_part, float* lse_t) {
  const long long total = static_cast<long long>(B) * Sq * Hq * 16;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  if (v && B != 1) return hipErrorInvalidValue;  // a varlen batch passes B = 1, Sq = total_q
  hipLaunchKernelGGL(combine_slots_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, o_part, lse_part, q2k, B, Sq, Hq, Hkv, topk, nblk,
                     v ? v->q_rows : nullptr, o, lse, lse_t_part, lse_t);
  return hipGetLastError();
}

hipError_t launch_combine_splits(const float* o_part, const float* lse_part, int B, int Sq, int Hq,
                                 int splits, uint16_t* o, float* lse, hipStream_t stream,
                                 const float* lse_t_part, float* lse_t) {
  const long long total = static_cast<long long>(B) * Sq * Hq * 16;
  const long long blocks = (total + 255) / 256;
  if (blocks > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(combine_splits_kernel, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     stream, o_part, lse_part, B, Sq, Hq, splits, o, lse, lse_t_part, lse_t);
  return hipGetLastError();
}

}  // namespace msa
