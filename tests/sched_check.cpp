// CPU driver of the host work distribution (segkv_sched.h).  No argument:
// the prefill work balancing; reads "n_bins n cost_0 .. cost_{n-1}" from
// stdin and prints the bin offsets and the grouped order, one line each.
// Argument "decode": the decode share cut; reads "n_wg piece_cost n len_0 ..
// len_{n-1}" and prints the share boundaries.
#include <cstdio>
#include <string>
#include <vector>

#include "segkv_sched.h"

static int decode_bounds() {
  long n_wg = 0, piece_cost = 0, n = 0;
  if (std::scanf("%ld %ld %ld", &n_wg, &piece_cost, &n) != 3) return 1;
  std::vector<int32_t> len(static_cast<size_t>(n));
  int64_t total = 0;
  for (auto &l : len) {
    if (std::scanf("%d", &l) != 1) return 1;
    total += l;
  }
  for (int64_t v : segkv::decode_share_bounds(len, total, n_wg, piece_cost)) std::printf("%ld ", static_cast<long>(v));
  std::printf("\n");
  return 0;
}

int main(int argc, char **argv) {
  if (argc > 1 && std::string(argv[1]) == "decode") return decode_bounds();
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
