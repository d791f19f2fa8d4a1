/*
 * Seeded synthetic inputs for top-k block-sparse attention workloads.
 *
 * Host-only C, shared by the tests, the benchmark and the CPU oracle's
 * callers. It holds no attention arithmetic: only random numbers and the
 * index-table recipes of the workloads (which blocks a query row selects).
 *
 * Random numbers come from a counter-based generator: the splitmix64 output
 * function (Steele, Lea and Flood, "Fast splittable pseudorandom number
 * generators", OOPSLA 2014) applied to key + (counter + 1) * golden-gamma.
 * Every element is a pure function of (seed, stream, counter), so any slice
 * is reproducible and the result does not depend on the thread count.
 *
 * Normals use the Box-Muller transform; uniform integers in [0, n) use the
 * multiply-high reduction of a 32-bit draw (Lemire, "Fast random integer
 * generation in an interval", 2019), whose tiny bias is irrelevant here.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GOLDEN_GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t sm64_mix(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

/* Key of an independent sub-stream of one seed. */
static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return sm64_mix(sm64_mix(seed + GOLDEN_GAMMA) ^ (stream * 0xD1B54A32D192ED03ULL + 1));
}

static inline uint64_t draw64(uint64_t key, uint64_t counter) {
  return sm64_mix(key + (counter + 1) * GOLDEN_GAMMA);
}

static inline uint32_t uniform_below(uint64_t key, uint64_t counter, uint32_t n) {
  uint32_t r = (uint32_t)(draw64(key, counter) >> 32);
  return (uint32_t)(((uint64_t)r * n) >> 32);
}

/* fp32 -> bf16 bit pattern, round to nearest even (inputs are finite). */
static inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

uint64_t wl_stream_key(uint64_t seed, uint64_t stream) { return stream_key(seed, stream); }
uint64_t wl_draw64(uint64_t key, uint64_t counter) { return draw64(key, counter); }

/* N(0,1) values rounded to bf16, elements [first, first + n) of a stream. */
void wl_normal_bf16(uint64_t seed, uint64_t stream, int64_t first, int64_t n, uint16_t* out) {
  const uint64_t key = stream_key(seed, stream);
  const double two_pi = 6.283185307179586476925286766559;
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) {
    const int64_t e = first + i;
    const uint64_t h = draw64(key, (uint64_t)(e >> 1));
    const double u1 = ((double)(h >> 32) + 0.5) * (1.0 / 4294967296.0);
    const double u2 = ((double)(h & 0xFFFFFFFFu) + 0.5) * (1.0 / 4294967296.0);
    const double r = sqrt(-2.0 * log(u1));
    const double z = (e & 1) ? r * sin(two_pi * u2) : r * cos(two_pi * u2);
    out[i] = f32_to_bf16_rne((float)z);
  }
}

/* Index-row recipes. */
enum { WL_PERM = 0, WL_SINK = 1, WL_CAUSAL = 2 };

static void sort_small(int32_t* a, int n) {
  for (int i = 1; i < n; ++i) {
    int32_t x = a[i];
    int j = i - 1;
    while (j >= 0 && a[j] > x) { a[j + 1] = a[j]; --j; }
    a[j + 1] = x;
  }
}

/* k distinct values from [lo, lo + n) by Floyd's sampling; draws use counters
 * base .. base + k - 1. */
static void floyd_sample(uint64_t key, uint64_t base, int32_t lo, int32_t n, int k, int32_t* out) {
  int cnt = 0;
  for (int32_t j = n - k; j < n; ++j) {
    int32_t t = (int32_t)uniform_below(key, base + (uint64_t)cnt, (uint32_t)(j + 1));
    int seen = 0;
    for (int i = 0; i < cnt; ++i) if (out[i] == lo + t) { seen = 1; break; }
    out[cnt++] = seen ? lo + j : lo + t;
  }
}

/* floor(a / b) for b > 0. */
static inline int64_t floor_div(int64_t a, int64_t b) {
  int64_t q = a / b;
  return (a % b != 0 && a < 0) ? q - 1 : q;
}

/*
 * q2k table [B, Hkv, Sq, topk] (int32, -1 = unused slot).
 *   WL_PERM:   the first topk entries of a random permutation of 0..nblk_b-1
 *              (permutation order, unsorted).
 *   WL_SINK:   block 0 plus topk-1 distinct blocks from 1..nblk_b-1, sorted.
 *   WL_CAUSAL: visible = clamp(floor((q + kvlen_b - Sq) / blk) + 1, 0, nblk_b);
 *              visible <= topk: 0..visible-1 then -1 padding; otherwise the
 *              diagonal block visible-1 plus topk-1 distinct blocks from
 *              0..visible-2, sorted.
 * kvlen[b] is the KV length of sequence b and nblk_b = ceil(kvlen[b] / blk).
 * Returns 0, or -1 on bad arguments.
 */
int wl_q2k(uint64_t seed, uint64_t stream, int mode, int B, int Hkv, int Sq, const int32_t* kvlen,
           int blk, int topk, int32_t* out) {
  if (B <= 0 || Hkv <= 0 || Sq <= 0 || blk <= 0 || topk <= 0 || topk > 64) return -1;
  for (int b = 0; b < B; ++b) {
    int64_t nb = ((int64_t)kvlen[b] + blk - 1) / blk;
    if (mode != WL_CAUSAL && nb < topk) return -1;
  }
  const uint64_t key = stream_key(seed, stream);
  const int64_t rows = (int64_t)B * Hkv * Sq;
#pragma omp parallel for schedule(static)
  for (int64_t r = 0; r < rows; ++r) {
    const int b = (int)(r / ((int64_t)Hkv * Sq));
    const int q = (int)(r % Sq);
    const int32_t nblk = (int32_t)(((int64_t)kvlen[b] + blk - 1) / blk);
    int32_t* row = out + r * topk;
    const uint64_t base = (uint64_t)r * 128u;
    if (mode == WL_PERM) {
      /* partial Fisher-Yates over 0..nblk-1, tracking only displaced entries */
      int32_t pos_val[64], pos_idx[64];
      int nmap = 0;
      for (int i = 0; i < topk; ++i) {
        int32_t j = i + (int32_t)uniform_below(key, base + (uint64_t)i, (uint32_t)(nblk - i));
        int32_t vi = i, vj = j;
        for (int m = 0; m < nmap; ++m) { if (pos_idx[m] == i) vi = pos_val[m]; if (pos_idx[m] == j) vj = pos_val[m]; }
        row[i] = vj;
        /* record a[j] = old a[i] */
        int found = 0;
        for (int m = 0; m < nmap; ++m) if (pos_idx[m] == j) { pos_val[m] = vi; found = 1; }
        if (!found) { pos_idx[nmap] = j; pos_val[nmap] = vi; ++nmap; }
      }
    } else if (mode == WL_SINK) {
      row[0] = 0;
      floyd_sample(key, base, 1, nblk - 1, topk - 1, row + 1);
      sort_small(row, topk);
    } else {
      int64_t vis = floor_div((int64_t)q + kvlen[b] - Sq, blk) + 1;
      if (vis < 0) vis = 0;
      if (vis > nblk) vis = nblk;
      if (vis <= topk) {
        for (int i = 0; i < topk; ++i) row[i] = i < vis ? i : -1;
      } else {
        row[0] = (int32_t)vis - 1;
        floyd_sample(key, base, 0, (int32_t)vis - 1, topk - 1, row + 1);
        sort_small(row, topk);
      }
    }
  }
  return 0;
}

/* A uniformly random permutation of 0..n-1 (Fisher-Yates). */
void wl_permutation(uint64_t seed, uint64_t stream, int64_t n, int32_t* out) {
  const uint64_t key = stream_key(seed, stream);
  for (int64_t i = 0; i < n; ++i) out[i] = (int32_t)i;
  for (int64_t i = n - 1; i > 0; --i) {
    int64_t j = (int64_t)uniform_below(key, (uint64_t)i, (uint32_t)(i + 1));
    int32_t t = out[i]; out[i] = out[j]; out[j] = t;
  }
}
