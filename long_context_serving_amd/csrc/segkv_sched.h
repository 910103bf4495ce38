// Host-side work distribution (no device types), header-only so that a CPU
// test can drive it directly: the static balancing of prefill work items over
// the resident workgroups, and the cut of the decode's stream-K page list
// into shares.
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

// Boundaries of n_wg contiguous shares of a list of segments laid end to end
// (len[i] >= 1 pages each, total = their sum), such that each share's cost,
// its pages plus piece_cost for every segment piece it holds, is about the
// same.  bounds[w] .. bounds[w + 1] is share w's page range; bounds[0] = 0,
// bounds[n_wg] = total, non-decreasing.  piece_cost = 0 gives equal page
// counts.  Shares are filled in order up to cumulative cost targets (w + 1) T,
// a new piece only where at least one page fits after its cost; T is found
// by bisection so that the last share's cost matches it.
inline std::vector<int64_t> decode_share_bounds(const std::vector<int32_t> &len, int64_t total, int64_t n_wg,
                                                int64_t piece_cost) {
  std::vector<int64_t> b(static_cast<size_t>(n_wg) + 1, total);
  b[0] = 0;
  for (int64_t w = 1; w < n_wg; ++w) b[static_cast<size_t>(w)] = total * w / n_wg;
  if (piece_cost <= 0 || n_wg <= 1 || len.empty()) return b;
  std::vector<int64_t> t(b.size(), total);
  t[0] = 0;
  // Fills shares 0 .. n_wg - 2; returns the last share's cost minus T.
  auto fill = [&](double T) -> double {
    size_t si = 0;
    int64_t seg_start = 0, pos = 0;
    double used = 0.0;  // cost of the pages and pieces placed so far
    for (int64_t w = 0; w + 1 < n_wg; ++w) {
      const double target = static_cast<double>(w + 1) * T;
      while (pos < total) {
        while (seg_start + len[si] <= pos) seg_start += len[si++];
        const int64_t rem = seg_start + len[si] - pos;
        const double room = target - used - static_cast<double>(piece_cost);
        if (room < 1.0) break;
        const int64_t take = std::min<int64_t>(rem, static_cast<int64_t>(room));
        pos += take;
        used += static_cast<double>(piece_cost + take);
        if (take < rem) break;
      }
      t[static_cast<size_t>(w) + 1] = pos;
    }
    int64_t pieces = 0;
    int64_t s0 = 0;
    for (int32_t l : len) {
      if (s0 + l > pos) ++pieces;
      s0 += l;
    }
    return static_cast<double>((total - pos) + piece_cost * pieces) - T;
  };
  double lo = static_cast<double>(total) / static_cast<double>(n_wg);
  double hi = static_cast<double>(total + piece_cost * (static_cast<int64_t>(len.size()) + n_wg));
  for (int it = 0; it < 60; ++it) {  // least T whose last share costs at most T
    const double mid = 0.5 * (lo + hi);
    if (fill(mid) <= 0.0)
      hi = mid;
    else
      lo = mid;
  }
  fill(hi);
  return t;
}

}  // namespace segkv
