// Host check of msa::kv_item_slot, the fixed slot of each kv-centric work item in the
// unsorted item table: reads "Hkv chunk_shift nrows" and then Hkv * nrows row lengths
// from stdin, and prints, for every chunk of every row (rows laid out back to back per
// KV head, as in a CSR), its slot and the table's slots per KV head. The test checks
// that the slots are distinct and below Hkv * per_head.
#include "../../block_sparse_attention_top_amd/csrc/msa_internal.hpp"

#include <stdio.h>

#include <vector>

int main() {
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
