// CPU driver of the in-page layout of the K and V pools (page_layout.h):
// prints, for head dim D and page size P given on the command line, the
// element offset of every 16-byte chunk of a K page (row-major over rows
// and chunks) and then of a V^T page (over channel rows and chunks).
#include <cstdio>
#include <cstdlib>

#define __device__
#define __forceinline__ inline
#include "page_layout.h"

template <int D, int P>
static void dump() {
  using PL = segkv::PageLayout<D, P>;
  for (int r = 0; r < P; ++r)
    for (int c = 0; c < D / 8; ++c) std::printf("%d ", PL::k_elem(r, c));
  std::printf("\n");
  for (int d = 0; d < D; ++d)
    for (int c = 0; c < P / 8; ++c) std::printf("%d ", PL::v_elem(d, c));
  std::printf("\n");
}

int main(int argc, char **argv) {
  if (argc != 3) return 1;
  const int D = std::atoi(argv[1]), P = std::atoi(argv[2]);
  if (D == 64 && P == 16) dump<64, 16>();
  else if (D == 64 && P == 32) dump<64, 32>();
  else if (D == 64 && P == 64) dump<64, 64>();
  else if (D == 128 && P == 16) dump<128, 16>();
  else if (D == 128 && P == 32) dump<128, 32>();
  else if (D == 128 && P == 64) dump<128, 64>();
  else return 2;
  return 0;
}
