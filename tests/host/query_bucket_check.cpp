// Host check of msa::query_bucket, the query-range bucketing of the kv-centric item
// order: prints floor(q * buckets / nq) (clamped) for each "q nq buckets" triple read
// from stdin. The test compares every line with exact integer arithmetic.
#include "../../block_sparse_attention_top_amd/csrc/msa_internal.hpp"

#include <stdio.h>

int main() {
  long long q, nq;
  int buckets;
  while (scanf("%lld %lld %d", &q, &nq, &buckets) == 3)
    printf("%d\n", msa::query_bucket(q, nq, buckets));
  return 0;
}
