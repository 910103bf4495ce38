// Static balancing of prefill work items over the resident workgroups (host
// code, no device types): each item, taken in the given order, goes to the
// workgroup with the least assigned cost so far (ties to the lowest index).
// Header-only so that a CPU test can drive it directly.
#pragma once

#include <stdint.h>

#include <algorithm>
#include <functional>
#include <utility>
#include <vector>

namespace segkv {

// cost[i] > 0 for i < n; n_bins >= 1.  On return bin_off[b] .. bin_off[b + 1]
// is bin b's range in `order`, and order lists the item indices bin by bin,
// each bin's items in their given order.  owner[i] is item i's bin.
inline void balance_items(const std::vector<int64_t> &cost, int32_t n_bins, std::vector<int32_t> *owner,
                          std::vector<int32_t> *bin_off, std::vector<int32_t> *order) {
  const size_t n = cost.size();
  owner->assign(n, 0);
  bin_off->assign(static_cast<size_t>(n_bins) + 1, 0);
  order->assign(n, 0);
  // min-heap of (assigned cost, bin)
  std::vector<std::pair<int64_t, int32_t>> heap;
  heap.reserve(static_cast<size_t>(n_bins));
  for (int32_t b = 0; b < n_bins; ++b) heap.emplace_back(0, b);
  const auto later = std::greater<std::pair<int64_t, int32_t>>();
  std::make_heap(heap.begin(), heap.end(), later);
  for (size_t i = 0; i < n; ++i) {
    std::pop_heap(heap.begin(), heap.end(), later);
    const int32_t b = heap.back().second;  // read before push_heap moves the element
    heap.back().first += cost[i];
    std::push_heap(heap.begin(), heap.end(), later);
    (*owner)[i] = b;
    (*bin_off)[static_cast<size_t>(b) + 1]++;
  }
  for (int32_t b = 0; b < n_bins; ++b) (*bin_off)[static_cast<size_t>(b) + 1] += (*bin_off)[static_cast<size_t>(b)];
  std::vector<int32_t> fill(bin_off->begin(), bin_off->end() - 1);
  for (size_t i = 0; i < n; ++i) (*order)[static_cast<size_t>(fill[static_cast<size_t>((*owner)[i])]++)] = static_cast<int32_t>(i);
}

}  // namespace segkv
