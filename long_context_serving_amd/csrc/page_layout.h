// Byte layout of one K page and one V^T page of the pools (device side).
//
// A K page holds P key rows of D bf16 channels; a V page holds the same
// keys transposed, D channel rows of P keys.  Within a page the rows are
// taken in pairs (2m, 2m+1), and each 128-byte line of the page holds the
// same 64-byte group of both rows of a pair: line (m, g) = [row 2m, group
// g][row 2m+1, group g].  V^T pages with channel rows of at most 64 bytes
// (P <= 32) are already laid out that way when stored row-major, and are.
//
// The point is the decode's operand loads.  A 16x16x32 MFMA operand takes
// one row per lane of a 16-lane group and 16 bytes of it per group, so one
// load instruction reads 64 bytes of each of 16 rows.  In a row-major page
// that is half of 16 lines, and the other half comes in a later instruction;
// lines fetched for the first half are often fetched again for the second
// (13% more memory reads in a probe of the pattern).  With rows interleaved
// in pairs, the 16 rows of an instruction are 8 pairs and each of its lines
// is read whole.  The prefill and score tile copies read 4 whole K rows
// (or 8 V^T rows) per instruction, 1 KiB that stays contiguous here.
#pragma once

namespace segkv {

template <int D, int P>
struct PageLayout {
  static_assert(P % 2 == 0 && D % 32 == 0, "rows pair up and split into 64-byte groups");
  static constexpr int K_CPR = D / 8;  // 16-byte chunks per K row
  static constexpr int V_CPR = P / 8;  // 16-byte chunks per V^T channel row
  // Element offset of 16-byte chunk c (channels 8c .. 8c+7) of K row `row`.
  static __device__ __forceinline__ int k_elem(int row, int c) {
    return ((((row >> 1) * (K_CPR / 4) + (c >> 2)) * 8) + (row & 1) * 4 + (c & 3)) * 8;
  }
  // Element offset of 16-byte chunk c (keys 8c .. 8c+7) of V^T channel row d.
  static __device__ __forceinline__ int v_elem(int d, int c) {
    if constexpr (V_CPR <= 4) {
      return d * P + c * 8;
    } else {
      return ((((d >> 1) * (V_CPR / 4) + (c >> 2)) * 8) + (d & 1) * 4 + (c & 3)) * 8;
    }
  }
};

}  // namespace segkv
