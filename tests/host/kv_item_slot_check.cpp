// Host check of msa::kv_item_slot, the fixed slot of each kv-centric work item in the
// unsorted item table, and of msa::kv_row_ok, the check a caller's CSR row passes
// before its items are listed. Two modes, chosen by the first word on stdin:
//
//   len Hkv chunk_shift nrows, then Hkv * nrows row lengths: rows laid out back to
//       back per KV head, as in a CSR; prints the table's slots per KV head, then the
//       slot of every chunk of every row.
//   ptr Hkv chunk_shift nrows cap, then Hkv * (nrows + 1) row_ptr values (any values,
//       as a caller might pass): prints the slots per KV head, whether some row failed
//       kv_row_ok (the item order is then void), and for every chunk of every row that
//       passed, as the item kernel lists it: its slot, first entry and end.
//
// The test checks that the slots fit the table, that every listed entry lies in
// [0, cap), and, when no row failed, that the slots are distinct.
#include "../../block_sparse_attention_top_amd/csrc/msa_internal.hpp"

#include <stdio.h>
#include <string.h>

#include <vector>

static int run_len() {
  int Hkv, shift, nrows;
  if (scanf("%d %d %d", &Hkv, &shift, &nrows) != 3) return 1;
  std::vector<long long> len(static_cast<size_t>(Hkv) * nrows);
  for (auto& x : len)
    if (scanf("%lld", &x) != 1) return 1;
  // per_head as the library sizes it: cap / chunk + nrows + 1, with cap >= every
  // KV head's entry count
  long long cap = 0;
  for (int h = 0; h < Hkv; ++h) {
    long long n = 0;
    for (int r = 0; r < nrows; ++r) n += len[static_cast<size_t>(h) * nrows + r];
    if (n > cap) cap = n;
  }
  const long long per_head = (cap >> shift) + nrows + 1;
  printf("%lld\n", per_head);
  for (int h = 0; h < Hkv; ++h) {
    long long beg = 0;
    for (int r = 0; r < nrows; ++r) {
      const long long n = len[static_cast<size_t>(h) * nrows + r];
      for (long long p = beg; p < beg + n; p += (1LL << shift))
        printf("%lld\n", msa::kv_item_slot(h, per_head, static_cast<int>(p), shift, r));
      beg += n;
    }
  }
  return 0;
}

static int run_ptr() {
  int Hkv, shift, nrows;
  long long cap;
  if (scanf("%d %d %d %lld", &Hkv, &shift, &nrows, &cap) != 4) return 1;
  std::vector<long long> rp(static_cast<size_t>(Hkv) * (nrows + 1));
  for (auto& x : rp)
    if (scanf("%lld", &x) != 1) return 1;
  const long long per_head = (cap >> shift) + nrows + 1;
  bool bad = false;
  for (int h = 0; h < Hkv; ++h)
    for (int r = 0; r < nrows; ++r) {
      const long long* p = &rp[static_cast<size_t>(h) * (nrows + 1) + r];
      if (!msa::kv_row_ok(p[0], p[1], cap)) bad = true;
    }
  printf("%lld %d\n", per_head, bad ? 1 : 0);
  for (int h = 0; h < Hkv; ++h)
    for (int r = 0; r < nrows; ++r) {
      const long long* p = &rp[static_cast<size_t>(h) * (nrows + 1) + r];
      if (!msa::kv_row_ok(p[0], p[1], cap)) continue;
      for (long long e = p[0]; e < p[1]; e += (1LL << shift)) {
        const long long end = e + (1LL << shift) < p[1] ? e + (1LL << shift) : p[1];
        printf("%lld %lld %lld\n", msa::kv_item_slot(h, per_head, static_cast<int>(e), shift, r),
               e, end);
      }
    }
  return 0;
}

int main() {
  char mode[8];
  if (scanf("%7s", mode) != 1) return 1;
  if (strcmp(mode, "len") == 0) return run_len();
  if (strcmp(mode, "ptr") == 0) return run_ptr();
  return 1;
}
