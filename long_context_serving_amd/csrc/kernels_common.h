// Device-side helpers shared by the HIP kernels of libsegkv (gfx950, CDNA4):
// vector types, bf16 packing, the query relocation, direct global->LDS
// copies, scalar table loads and the LDS layout of a prefill K/V tile.
//
// The attention computed is masked softmax attention in which each KV head
// sees either the full causal context (global) or a sliding window of its W
// most recent tokens (local) ("Xiaohongshu Open-Sources RedKnot" page,
// section "What Happened", items 1 and 3).  No mask is materialised: each
// workgroup only visits the KV tiles its rows can see, and only tiles that
// straddle a window edge or the causal diagonal evaluate the per-key
// predicate.
//
// Pool layout (one page = page_size tokens of one (layer, sequence, KV head)):
//   K page  page_size key rows of head_dim channels
//   V page  head_dim channel rows of page_size keys (transposed)
// with rows stored in pairs, 64-byte groups interleaved (page_layout.h).
// Both operands of both products then load 16-byte runs straight into the
// MFMA operand layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "segkv_internal.h"

namespace segkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_inff();

// Softmax probabilities are exp2 of scaled, max-shifted scores.  v_exp_f32
// flushes results below 2^-126 to zero, which only drops terms far below
// the fp32 resolution of the row sum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// The running max of a row moves only when a tile's max exceeds it by more
// than this many powers of two, so most tiles skip rescaling the output
// accumulators.  Probabilities then stay <= 2^8 (exact in bf16's exponent
// range, and far from fp32 overflow in the sums).
constexpr float kRescaleLog2 = 8.0f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ u32x4 ld16(const uint16_t *p) { return *reinterpret_cast<const u32x4 *>(p); }

__device__ __forceinline__ u32x2 pack4_bf16(float a, float b, float c, float d) {
  bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ bf16x8 pack8_bf16(float a0, float a1, float a2, float a3, float a4, float a5, float a6,
                                             float a7) {
  bf16x8 v = {(__bf16)a0, (__bf16)a1, (__bf16)a2, (__bf16)a3, (__bf16)a4, (__bf16)a5, (__bf16)a6, (__bf16)a7};
  return v;
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __builtin_bit_cast(float, w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __builtin_bit_cast(float, w & 0xffff0000u); }

// Query-side RoPE relocation of channels ch0 .. ch0+7 of one query row
// ("RedKnot-MLA: Multi-Head Offline-Online Reuse for DeepSeek-V4 Long-Context
// Serving" review, "Summary"): channel c becomes cos[c] q[c] + ssin[c]
// q[partner(c)] in fp32 (tab = cos[D] then signed sin[D] of the segment's
// offset), rounded once to bf16.  ch0 is a multiple of 8.  The loaded data
// and the arithmetic are kept apart so that several chunks' loads (BATCH) can
// be in flight before the first rotation.
struct RelocIn {
  u32x4 x, y;         // the chunk and its partner chunk (bf16 pairs)
  f32x4 c0, c1, s0, s1;  // cos and signed sin of its 8 channels
};

__device__ __forceinline__ u32x4 reloc_apply(const RelocIn &in, const RopeArgs &r) {
  const float cs[8] = {in.c0[0], in.c0[1], in.c0[2], in.c0[3], in.c1[0], in.c1[1], in.c1[2], in.c1[3]};
  const float sn[8] = {in.s0[0], in.s0[1], in.s0[2], in.s0[3], in.s1[0], in.s1[1], in.s1[2], in.s1[3]};
  float out[8];
  const bool swap = r.style == 1;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float xl = bf16_lo(in.x[w]), xh = bf16_hi(in.x[w]);
    const float yl = bf16_lo(in.y[w]), yh = bf16_hi(in.y[w]);
    out[2 * w] = cs[2 * w] * xl + sn[2 * w] * (swap ? yh : yl);
    out[2 * w + 1] = cs[2 * w + 1] * xh + sn[2 * w + 1] * (swap ? yl : yh);
  }
  return __builtin_bit_cast(u32x4, pack8_bf16(out[0], out[1], out[2], out[3], out[4], out[5], out[6], out[7]));
}

// Relocated Q operand chunks kk = 0 .. NKK-1 of one row (chunk kk starts at
// channel kk * step + off); rows that are not valid get zeros.  The
// segment's cos/sin table is first copied into this wave's LDS (wtab, 2 * D
// floats; one coalesced 16-byte load per lane): every lane of a wave reads
// the same few table entries, which as vector loads from memory would be
// processed lane by lane, but as LDS reads are broadcasts.  A wave's own LDS
// operations complete in order, so no barrier is needed.  Four chunks' loads
// are in flight before the first rotation.
template <int D, int NKK, int BATCH = 4>
__device__ __forceinline__ void relocate_row(bf16x8 (&qv)[NKK], const uint16_t *qrow, int step, int off, bool valid,
                                             const float *tab, float *wtab, const RopeArgs &r) {
  constexpr int B = NKK < BATCH ? NKK : BATCH;
  static_assert(NKK % B == 0, "chunk batches");
  const int lane = threadIdx.x & 63;
  for (int i = lane; i < D / 2; i += 64)
    *reinterpret_cast<f32x4 *>(wtab + 4 * i) = *reinterpret_cast<const f32x4 *>(tab + 4 * i);
  const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int k0 = 0; k0 < NKK; k0 += B) {
    RelocIn in[B];
#pragma unroll
    for (int j = 0; j < B; ++j) {
      const int ch0 = (k0 + j) * step + off;
      int pc = ch0;
      if (r.style == 0 && ch0 >= r.lo) pc = ch0 - r.lo < r.half ? ch0 + r.half : ch0 - r.half;
      in[j].x = ld16(qrow + ch0);
      in[j].y = ld16(qrow + pc);
      in[j].c0 = *reinterpret_cast<const f32x4 *>(wtab + ch0);
      in[j].c1 = *reinterpret_cast<const f32x4 *>(wtab + ch0 + 4);
      in[j].s0 = *reinterpret_cast<const f32x4 *>(wtab + D + ch0);
      in[j].s1 = *reinterpret_cast<const f32x4 *>(wtab + D + ch0 + 4);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < B; ++j) qv[k0 + j] = as_bf16x8(valid ? reloc_apply(in[j], r) : z);
  }
}


// ===========================================================================
// Prefill layout (all prefill and score kernels).
//
// Products are done transposed, S^T = K Q^T and O^T += V^T P^T, with the
// gfx950 MFMA v_mfma_f32_32x32x16_bf16 (wave64; lane l holds operand row
// l % 32 and k-elements 8*(l / 32) .. +7; result lane l holds column l % 32
// and rows 8*(v/4) + 4*(l/32) + v%4 of register v).  A column is one query
// row, so the softmax statistics of a row live in one lane pair (l, l^32).
// The rows of the 32-key S^T blocks are mapped to keys so that the eight
// probabilities a lane feeds to the PV product belong to 8 consecutive keys:
// S^T row 8i + 4h + j of block kb holds key 32 kb + 16 (i/2) + 8 h + 4 (i%2)
// + j, hence register v of lane half h holds key 16 (v/8) + 8 h + v%8.
// ===========================================================================

__device__ __forceinline__ int st_row_key(int r) {  // S^T row -> key within a 32-key block
  const int i = r >> 3, h = (r >> 2) & 1, j = r & 3;
  return ((i >> 1) << 4) + (h << 3) + ((i & 1) << 2) + j;
}

// Max and sum of the 32 scores a lane holds for one column, as trees
// (3-input max; four independent add chains).
__device__ __forceinline__ float max32(const f32x16 &x, const f32x16 &y) {
  float r[11];
#pragma unroll
  for (int i = 0; i < 5; ++i) r[i] = fmaxf(fmaxf(x[3 * i], x[3 * i + 1]), x[3 * i + 2]);
  r[5] = fmaxf(fmaxf(x[15], y[0]), y[1]);
#pragma unroll
  for (int i = 0; i < 4; ++i) r[6 + i] = fmaxf(fmaxf(y[2 + 3 * i], y[3 + 3 * i]), y[4 + 3 * i]);
  r[10] = fmaxf(y[14], y[15]);
  const float a = fmaxf(fmaxf(r[0], r[1]), r[2]);
  const float b = fmaxf(fmaxf(r[3], r[4]), r[5]);
  const float c = fmaxf(fmaxf(r[6], r[7]), r[8]);
  return fmaxf(fmaxf(a, b), fmaxf(fmaxf(c, r[9]), r[10]));
}

__device__ __forceinline__ float sum32(const f32x16 &x, const f32x16 &y) {
  float s0 = x[0] + x[1], s1 = x[2] + x[3], s2 = y[0] + y[1], s3 = y[2] + y[3];
#pragma unroll
  for (int i = 4; i < 16; i += 4) {
    s0 += x[i] + x[i + 1];
    s1 += x[i + 2] + x[i + 3];
    s2 += y[i] + y[i + 1];
    s3 += y[i + 2] + y[i + 3];
  }
  return (s0 + s1) + (s2 + s3);
}

// Direct global->LDS copy of 16 bytes per lane (gfx950 global_load_lds_dwordx4):
// lane i writes bytes [16 i, 16 i + 16) after the wave-uniform LDS address
// lds_dst (taken from M0).  Completion is tracked by vmcnt, and every caller
// waits for it explicitly (s_waitcnt vmcnt(N) before the barrier that
// publishes a tile).  Issued as asm so that the compiler does not add its
// own wait for all outstanding LDS copies before each LDS read: it cannot
// tell the stage being read from the stages still loading, and would
// drain the prefetch.  The asm has no output registers; the LDS address
// escapes through it, so reads of the tiles are not folded away.
__device__ __forceinline__ void lds_dma16(const void *src, void *lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_dst)));
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(m0));
}

// The same copy with the source given as a wave-uniform base (SGPRs) plus a
// per-lane 32-bit byte offset (global_load_lds_dwordx4's saddr form): the
// address arithmetic per tile is then scalar.
__device__ __forceinline__ void lds_dma16_s(const void *sbase, uint32_t voff, void *lds_dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_dst)));
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(m0));
}

// Load of a per-call table entry (4, 16 or 32 bytes at a wave-uniform,
// 4-byte aligned address; no kernel writes these tables) through the scalar
// cache.  Written as asm because the compiler turns such reads into vector
// loads once the kernel stores to global memory, and a vector load's wait
// also waits for every tile load issued before it (vector loads complete in
// issue order).  The asm waits for its own result; lgkmcnt also covers this
// wave's outstanding LDS operations.
template <typename T>
__device__ __forceinline__ T sload(const T *q) {
  static_assert(sizeof(T) == 4 || sizeof(T) == 16 || sizeof(T) == 32, "scalar table loads are 1, 4 or 8 dwords");
  // The address is wave-uniform at every call; reading it from the first
  // lane lets it sit in SGPRs even where the compiler cannot prove that.
  const uint64_t a = reinterpret_cast<uint64_t>(q);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32)));
  const T *p = reinterpret_cast<const T *>(lo | (hi << 32));
  if constexpr (sizeof(T) == 32) {
    i32x8 v;
    asm volatile("s_load_dwordx8 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
    return __builtin_bit_cast(T, v);
  } else if constexpr (sizeof(T) == 16) {
    i32x4 v;
    asm volatile("s_load_dwordx4 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
    return __builtin_bit_cast(T, v);
  } else {
    int32_t v;
    asm volatile("s_load_dword %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(v) : "s"(p));
    return __builtin_bit_cast(T, v);
  }
}

// LDS layout of one prefill stage: the K tile (64 keys x D) and then the V^T
// tile (D channels x 64 keys), both unpadded with 16-byte chunks XOR-swizzled
// per row, so that every 16-lane phase of a ds_read_b128 of either MFMA
// operand touches 16 distinct bank groups, and so that the tiles can be
// filled by direct global->LDS loads (each lane of a wave writes the next 16
// bytes of a contiguous 1 KiB run).
template <int D>
struct PrefillLds {
  static constexpr int KCPR = D / 8;                       // 16-byte chunks per K row
  static constexpr int K_CHUNKS = kTileKeys * KCPR;
  static constexpr int V_CHUNKS = D * (kTileKeys / 8);
  static constexpr int STAGE_BYTES = (K_CHUNKS + V_CHUNKS) * 16;
  // Rows sharing one 256-byte bank cycle differ in their swizzle.
  static __device__ __forceinline__ int k_swz(int row) { return KCPR == 16 ? (row & 15) : ((row >> 1) & 7); }
  static __device__ __forceinline__ int v_swz(int row) { return (row >> 1) & 7; }
  static __device__ __forceinline__ int k_chunk(int key, int c) { return key * KCPR + (c ^ k_swz(key)); }
  static __device__ __forceinline__ int v_chunk(int d, int c) { return K_CHUNKS + d * 8 + (c ^ v_swz(d)); }
};

}  // namespace
}  // namespace segkv

// Launch of KERNEL<D, P> for the supported (head_dim, page_size) pairs; an
// unsupported pair returns hipErrorInvalidValue from the calling launcher.
#define SEGKV_DISPATCH_DP(KERNEL, D, P, GRID, BLOCK, STREAM, ARGS)                                \
  do {                                                                                           \
    if ((D) == 64 && (P) == 16) SEGKV_LAUNCH((KERNEL<64, 16>), GRID, BLOCK, STREAM, ARGS); \
    else if ((D) == 64 && (P) == 32) SEGKV_LAUNCH((KERNEL<64, 32>), GRID, BLOCK, STREAM, ARGS); \
    else if ((D) == 64 && (P) == 64) SEGKV_LAUNCH((KERNEL<64, 64>), GRID, BLOCK, STREAM, ARGS); \
    else if ((D) == 128 && (P) == 16) SEGKV_LAUNCH((KERNEL<128, 16>), GRID, BLOCK, STREAM, ARGS); \
    else if ((D) == 128 && (P) == 32) SEGKV_LAUNCH((KERNEL<128, 32>), GRID, BLOCK, STREAM, ARGS); \
    else if ((D) == 128 && (P) == 64) SEGKV_LAUNCH((KERNEL<128, 64>), GRID, BLOCK, STREAM, ARGS); \
    else return hipErrorInvalidValue;                                                            \
  } while (0)
