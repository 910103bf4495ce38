// HIP kernel of libsegkv: the head-decomposition merge.

#include "kernels_common.h"
#include "segkv_launch.h"

namespace segkv {
namespace {

// ===========================================================================
// Head-decomposition merge ("RedKnot: Head-Aware KV Reuse and
// SegPagedAttention" page, "The Three Core Mechanisms in Detail", first
// mechanism): each (row, head) pair takes the offline partial A, the online
// partial B, or their log-sum-exp merge over the union of their key sets.
// HBM streaming: D/8 lanes move one pair's 16-byte chunks, each lane keeps
// kMergeUnroll pairs in flight, and a pair reads only what its mode needs.
// A lane reads its chunk before it writes it, so o may alias o_a or o_b.
// ===========================================================================

template <int D>
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(MergeArgs a) {
  constexpr int LPP = D / 8;                // lanes per pair
  constexpr int PPW = kMergeThreads / LPP;  // pairs per workgroup pass
  constexpr int U = kMergeUnroll;
  static_assert(64 % LPP == 0, "a pair's lanes sit in one wave");
  const int sub = threadIdx.x % LPP;
  const int64_t n = a.n_pairs;
  const int64_t stride = static_cast<int64_t>(gridDim.x) * PPW * U;
  for (int64_t base = static_cast<int64_t>(blockIdx.x) * PPW * U + threadIdx.x / LPP; base < n; base += stride) {
    int md[U];
    float la[U], lb[U];
    u32x4 xa[U], xb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t i = base + static_cast<int64_t>(u) * PPW;
      md[u] = -1;
      la[u] = lb[u] = kNegInf;
      xa[u] = xb[u] = u32x4{0u, 0u, 0u, 0u};
      if (i < n) {
        md[u] = a.mode[i];
        if (md[u] != 1) {
          la[u] = a.lse_a[i];
          xa[u] = ld16(a.o_a + i * D + sub * 8);
        }
        if (md[u] != 0) {
          lb[u] = a.lse_b[i];
          xb[u] = ld16(a.o_b + i * D + sub * 8);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (md[u] < 0) continue;
      const int64_t i = base + static_cast<int64_t>(u) * PPW;
      u32x4 out;
      float l;
      if (md[u] == 0) {
        out = xa[u];
        l = la[u];
      } else if (md[u] == 1) {
        out = xb[u];
        l = lb[u];
      } else {
        const float m = fmaxf(la[u], lb[u]);
        if (m == kNegInf) {
          out = u32x4{0u, 0u, 0u, 0u};
          l = kNegInf;
        } else {
          const float wa = __expf(la[u] - m), wb = __expf(lb[u] - m);  // -inf parts give 0
          const float inv = 1.f / (wa + wb);
          const float ca = wa * inv, cb = wb * inv;
          float r[8];
#pragma unroll
          for (int w = 0; w < 4; ++w) {
            r[2 * w] = ca * bf16_lo(xa[u][w]) + cb * bf16_lo(xb[u][w]);
            r[2 * w + 1] = ca * bf16_hi(xa[u][w]) + cb * bf16_hi(xb[u][w]);
          }
          out = __builtin_bit_cast(u32x4, pack8_bf16(r[0], r[1], r[2], r[3], r[4], r[5], r[6], r[7]));
          l = m + logf(wa + wb);
        }
      }
      *reinterpret_cast<u32x4 *>(a.o + i * D + sub * 8) = out;
      if (sub == 0 && a.lse) a.lse[i] = l;
    }
  }
}

}  // namespace

hipError_t launch_merge(const MergeArgs &a, int n_wgs, int head_dim, hipStream_t s) {
  if (n_wgs <= 0 || a.n_pairs <= 0) return hipSuccess;
  if (head_dim == 64) SEGKV_LAUNCH(merge_kernel<64>, dim3(n_wgs), dim3(kMergeThreads), s, a);
  else if (head_dim == 128) SEGKV_LAUNCH(merge_kernel<128>, dim3(n_wgs), dim3(kMergeThreads), s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace segkv
