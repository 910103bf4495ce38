// CPU driver of the prefill work balancing (segkv_sched.h): reads
// "n_bins n cost_0 .. cost_{n-1}" from stdin and prints the bin offsets and
// the grouped order, one line each.
#include <cstdio>
#include <vector>

#include "segkv_sched.h"

int main() {
  int n_bins = 0;
  long n = 0;
  if (std::scanf("%d %ld", &n_bins, &n) != 2) return 1;
  std::vector<int64_t> cost(static_cast<size_t>(n));
  for (auto &c : cost)
    if (std::scanf("%ld", &c) != 1) return 1;
  std::vector<int32_t> owner, off, order;
  segkv::balance_items(cost, n_bins, &owner, &off, &order);
  for (int32_t v : off) std::printf("%d ", v);
  std::printf("\n");
  for (int32_t v : order) std::printf("%d ", v);
  std::printf("\n");
  return 0;
}
