// HIP kernels of libsegkv: KV append scatter and the per-call table upload.

#include "kernels_common.h"
#include "page_layout.h"
#include "segkv_launch.h"

namespace segkv {
namespace {

// ===========================================================================
// Scatter: copy newly appended K/V rows into their pages.
// ===========================================================================

template <int D, int P>
__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(ScatterArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sv[P * D];
  const int tid = threadIdx.x;
  if (static_cast<int>(blockIdx.x) < a.copy_wgs) {  // staged tables of the next call
    for (int i = blockIdx.x * kScatterThreads + tid; i < a.copy_n16; i += a.copy_wgs * kScatterThreads)
      a.copy_dst[i] = a.copy_src[i];
    return;
  }
  const ScatterItem it = a.items[blockIdx.x - a.copy_wgs];
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  using PL = PageLayout<D, P>;
  // 16-byte chunk c of staged V row `slot` sits at chunk c ^ (slot / 8 % CPR)
  auto vswz = [](int slot, int c) { return c ^ ((slot >> 3) & (CPR - 1)); };
  const int n_rows = it.slot_end - it.slot_begin;
  uint16_t *kpage = a.k_pool + static_cast<size_t>(it.page_id) * P * D;
  uint16_t *vpage = a.v_pool + static_cast<size_t>(it.page_id) * P * D;

  // Copy-on-write: slots [0, slot_begin) of the shared page this one
  // replaces.  They are disjoint from every slot written below.
  if (it.copy_from >= 0) {
    const uint16_t *ksrc = a.k_pool + static_cast<size_t>(it.copy_from) * P * D;
    const uint16_t *vsrc = a.v_pool + static_cast<size_t>(it.copy_from) * P * D;
    for (int c = tid; c < it.slot_begin * CPR; c += kScatterThreads) {
      const int off = PL::k_elem(c / CPR, c % CPR);
      *reinterpret_cast<u32x4 *>(kpage + off) = ld16(ksrc + off);
    }
    for (int c = tid; c < D * it.slot_begin; c += kScatterThreads) {
      const int d = c / it.slot_begin, sl = c - d * it.slot_begin;
      const int off = PL::v_elem(d, sl >> 3) + (sl & 7);
      vpage[off] = vsrc[off];
    }
  }

  // K rows, and V rows staged in LDS for the transpose.  All of a thread's
  // loads are issued before any store (the pools and the new rows may
  // alias as far as the compiler knows, so it would not batch them).
  constexpr int ITER = (P * CPR + kScatterThreads - 1) / kScatterThreads;
  u32x4 kx[ITER], vx[ITER];
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int c = tid + i * kScatterThreads;
    if (c < n_rows * CPR) {
      const int row = c / CPR, dc = c - row * CPR;
      const size_t src = (static_cast<size_t>(it.src_row + row) * a.num_kv_heads + it.kv_head) * D + dc * 8;
      kx[i] = ld16(a.k_new + src);
      vx[i] = ld16(a.v_new + src);
    }
  }
#pragma unroll
  for (int i = 0; i < ITER; ++i) {
    const int c = tid + i * kScatterThreads;
    if (c < n_rows * CPR) {
      const int row = c / CPR, dc = c - row * CPR;
      *reinterpret_cast<u32x4 *>(kpage + PL::k_elem(it.slot_begin + row, dc)) = kx[i];
      *reinterpret_cast<u32x4 *>(sv + (it.slot_begin + row) * D + vswz(it.slot_begin + row, dc) * 8) = vx[i];
    }
  }
  if (it.zero_tail) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int c = tid; c < (P - it.slot_end) * CPR; c += kScatterThreads) {
      const int row = c / CPR, dc = c - row * CPR;
      *reinterpret_cast<u32x4 *>(kpage + PL::k_elem(it.slot_end + row, dc)) = z;
      *reinterpret_cast<u32x4 *>(sv + (it.slot_end + row) * D + vswz(it.slot_end + row, dc) * 8) = z;
    }
  }
  __syncthreads();
  // V^T rows: channel d takes slots [slot_begin, wend).  A lane takes a
  // channel pair and 8 consecutive slots: one 4-byte LDS read per slot and
  // two 16-byte stores.  Consecutive lanes take consecutive slot groups of
  // one channel pair, so 8 lanes store both channel rows of the pair (whole
  // lines of the page); the chunk swizzle of the staged rows spreads their
  // LDS reads over the banks.
  const int wend = it.zero_tail ? P : it.slot_end;
  const int n = wend - it.slot_begin;
  if ((it.slot_begin & 7) == 0 && (n & 7) == 0) {
    constexpr int NPAIR = D / 2;
    const int groups = n / 8;
    for (int c = tid; c < NPAIR * groups; c += kScatterThreads) {
      const int dp = c / groups, s0 = it.slot_begin + (c % groups) * 8;
      uint32_t w[8];
#pragma unroll
      for (int e = 0; e < 8; ++e)
        w[e] = *reinterpret_cast<const uint32_t *>(sv + (s0 + e) * D + vswz(s0 + e, dp >> 2) * 8 + 2 * (dp & 3));
      u32x4 lo, hi;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        lo[e] = (w[2 * e] & 0xffffu) | (w[2 * e + 1] << 16);
        hi[e] = (w[2 * e] >> 16) | (w[2 * e + 1] & 0xffff0000u);
      }
      *reinterpret_cast<u32x4 *>(vpage + PL::v_elem(2 * dp, s0 >> 3)) = lo;
      *reinterpret_cast<u32x4 *>(vpage + PL::v_elem(2 * dp + 1, s0 >> 3)) = hi;
    }
  } else {
    for (int c = tid; c < D * n; c += kScatterThreads) {
      const int d = c / n, s = it.slot_begin + (c - d * n);
      vpage[PL::v_elem(d, s >> 3) + (s & 7)] = sv[s * D + vswz(s, d >> 3) * 8 + (d & 7)];
    }
  }
}

// Copy of the per-call tables from pinned host memory to device memory.
__global__ __launch_bounds__(256) void upload_kernel(uint4 *dst, const uint4 *src, size_t n16) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

}  // namespace

hipError_t launch_scatter(const ScatterArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(scatter_kernel, head_dim, page_size, dim3(n_items + a.copy_wgs), dim3(kScatterThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_upload(void *dst, const void *src_pinned, size_t bytes, hipStream_t s) {
  const size_t n16 = (bytes + 15) / 16;
  if (n16 == 0) return hipSuccess;
  SEGKV_LAUNCH(upload_kernel, dim3(static_cast<unsigned>((n16 + 255) / 256)), dim3(256), s,
               static_cast<uint4 *>(dst), static_cast<const uint4 *>(src_pinned), n16);
  return hipGetLastError();
}

}  // namespace segkv
