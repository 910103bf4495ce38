// HIP kernels of libsegkv for gfx950 (CDNA4): KV append scatter, varlen
// prefill attention, split-KV decode and the log-sum-exp combine.
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
//   K page  [page_size][head_dim]  row-major, a key row is contiguous
//   V page  [head_dim][page_size]  transposed, a channel row is contiguous
// Both operands of both products then load 16-byte runs straight into the
// MFMA operand layout.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
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
// and the arithmetic are kept apart so that several chunks' loads can be in
// flight before the first rotation.
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
template <int D, int NKK>
__device__ __forceinline__ void relocate_row(bf16x8 (&qv)[NKK], const uint16_t *qrow, int step, int off, bool valid,
                                             const float *tab, float *wtab, const RopeArgs &r) {
  constexpr int B = NKK < 4 ? NKK : 4;
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
    for (int c = tid; c < it.slot_begin * CPR; c += kScatterThreads)
      *reinterpret_cast<u32x4 *>(kpage + c * 8) = ld16(ksrc + c * 8);
    for (int c = tid; c < D * it.slot_begin; c += kScatterThreads) {
      const int d = c / it.slot_begin, sl = c - d * it.slot_begin;
      vpage[d * P + sl] = vsrc[d * P + sl];
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
      *reinterpret_cast<u32x4 *>(kpage + static_cast<size_t>(it.slot_begin + row) * D + dc * 8) = kx[i];
      *reinterpret_cast<u32x4 *>(sv + (it.slot_begin + row) * D + vswz(it.slot_begin + row, dc) * 8) = vx[i];
    }
  }
  if (it.zero_tail) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int c = tid; c < (P - it.slot_end) * CPR; c += kScatterThreads) {
      const int row = c / CPR, dc = c - row * CPR;
      *reinterpret_cast<u32x4 *>(kpage + static_cast<size_t>(it.slot_end + row) * D + dc * 8) = z;
      *reinterpret_cast<u32x4 *>(sv + (it.slot_end + row) * D + vswz(it.slot_end + row, dc) * 8) = z;
    }
  }
  __syncthreads();
  // V^T rows: channel d holds slots [slot_begin, wend) contiguously.  A
  // lane takes a channel pair and 8 consecutive slots: one 4-byte LDS read
  // per slot and two 16-byte stores.  Consecutive lanes take consecutive
  // slot groups of one channel pair, so 8 lanes store a whole 128-byte
  // channel row; the chunk swizzle of the staged rows spreads their LDS
  // reads over the banks.
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
      *reinterpret_cast<u32x4 *>(vpage + static_cast<size_t>(2 * dp) * P + s0) = lo;
      *reinterpret_cast<u32x4 *>(vpage + static_cast<size_t>(2 * dp + 1) * P + s0) = hi;
    }
  } else {
    for (int c = tid; c < D * n; c += kScatterThreads) {
      const int d = c / n, s = it.slot_begin + (c - d * n);
      vpage[static_cast<size_t>(d) * P + s] = sv[s * D + vswz(s, d >> 3) * 8 + (d & 7)];
    }
  }
}

// ===========================================================================
// Prefill: a persistent grid, one workgroup per CU.  Each workgroup takes
// work items from a queue in list order (longest first); an item is 256
// (query position, query head) rows of one (sequence, KV head group) over a
// range of 64-key tiles.  The K/V tile loads run two tiles ahead across item
// boundaries, so a workgroup never waits for its next item's first tiles.
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

template <int D, int P>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillArgs a) {
  using L = PrefillLds<D>;
  constexpr int NKK = D / 16;  // k-steps of the QK product
  constexpr int NDB = D / 32;  // 32-channel blocks of O^T
  constexpr int NW = kPrefillThreads / 64;
  constexpr int K_INSTR = L::K_CHUNKS / kPrefillThreads;  // direct loads per lane per tile (K)
  constexpr int V_INSTR = L::V_CHUNKS / kPrefillThreads;  // (V^T)
  constexpr int NSTAGE = 3;
  constexpr int LOADS_PER_TILE = K_INSTR + V_INSTR;
  static_assert(kPrefillRows == 32 * NW, "one 32-row column block per wave");
  static_assert(K_INSTR >= 1 && V_INSTR >= 1, "tile smaller than one load per lane");
  __shared__ __attribute__((aligned(16))) uint4 smem4[NSTAGE * L::STAGE_BYTES / 16];
  __shared__ int s_next[2];  // item indices fetched by thread 0; consecutive fetches alternate slots
  __shared__ __attribute__((aligned(16))) float s_rope[NW][2 * D];  // per-wave relocation table
  char *smem = reinterpret_cast<char *>(smem4);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int G = a.group;
  const int rows = a.rows_per_tile;
  const int n_items = a.n_items;
  const int r = wave * 32 + col;  // this lane's row of the item
  const int pos_off = r / G;

  // Work queue: each workgroup takes items in list order (longest first).
  // cur is being computed; nxt is the next item this workgroup owns (-1
  // while its index is still in flight through LDS).
  if (tid == 0) s_next[0] = atomicAdd(a.counter, 1);
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(s_next[0]);  // uniform: descriptors load through the scalar cache
  if (cur >= n_items) return;
  // The next item is taken late (three tiles before the current one ends),
  // so the list is handed out longest first; its index arrives through LDS.
  int nxt = -1;
  int fslot = 1;  // slot of the next fetch: a slot is rewritten only after every wave passed a later barrier

  // Producer: global->LDS tile loads run up to two tiles ahead of the
  // consumer along the sequence of this workgroup's items, so the next
  // item's first tiles load while the current one finishes.
  int p_item = -1, p_tile = 0, p_end = 0;  // next tile to issue (p_item < 0: waiting for nxt)
  SegDesc psg;
  auto p_set = [&](int idx) {  // point the producer at item idx (descriptors read once per item)
    const PrefillItem pi_ = sload(a.items + idx);
    p_item = idx;
    p_tile = pi_.tile_begin;
    p_end = pi_.tile_end;
    psg = sload(a.segs + pi_.seq * a.num_kv_heads + pi_.kv_head);
  };
  p_set(cur);
  int issued = 0, consumed = 0;                      // tiles issued / computed so far
  auto issue_tile = [&](int tile, int stage) {
    const int k0 = tile * kTileKeys;
    const int last_page = psg.n_pages - 1;
    char *st = smem + stage * L::STAGE_BYTES;
    // The tile's keys lie on NP whole pages (first_token is page aligned);
    // their ids are uniform, read by scalar loads.  Keys before the first
    // stored page or after the last one (never visible) read slot 0 of the
    // nearest stored page.
    constexpr int NP = kTileKeys / P;
    int pid[NP];
    const int pg0 = (k0 - psg.first_token) / P;
#pragma unroll
    for (int i = 0; i < NP; ++i) pid[i] = sload(a.page_ids + psg.page_off + min(max(pg0 + i, 0), last_page));
    auto page_of = [&](int key_in_tile, int *slot) {
      const int rel = k0 + key_in_tile - psg.first_token;
      *slot = rel >= 0 && rel / P <= last_page ? key_in_tile % P : 0;
      int page = pid[0];
#pragma unroll
      for (int i = 1; i < NP; ++i)
        if (key_in_tile / P == i) page = pid[i];
      return page;
    };
#pragma unroll
    for (int j = 0; j < K_INSTR; ++j) {
      const int c = (j * NW + wave) * 64 + lane;
      const int row = c / L::KCPR;
      const int logical = (c % L::KCPR) ^ L::k_swz(row);
      if constexpr (P == kTileKeys) {
        // one page per tile: a scalar page base and a 32-bit lane offset
        lds_dma16_s(a.k_pool + static_cast<size_t>(pid[0]) * (P * D), static_cast<uint32_t>((row * D + logical * 8) * 2),
                    st + (j * NW + wave) * 1024);
      } else {
        int slot;
        const int page = page_of(row, &slot);
        lds_dma16(a.k_pool + (static_cast<size_t>(page) * P + slot) * D + logical * 8, st + (j * NW + wave) * 1024);
      }
    }
#pragma unroll
    for (int j = 0; j < V_INSTR; ++j) {
      const int c = (j * NW + wave) * 64 + lane;
      const int d = c / 8;
      const int logical = (c % 8) ^ L::v_swz(d);
      if constexpr (P == kTileKeys) {
        lds_dma16_s(a.v_pool + static_cast<size_t>(pid[0]) * (P * D), static_cast<uint32_t>((d * P + logical * 8) * 2),
                    st + L::K_CHUNKS * 16 + (j * NW + wave) * 1024);
      } else {
        int slot;
        const int page = page_of(logical * 8, &slot);
        lds_dma16(a.v_pool + static_cast<size_t>(page) * (P * D) + d * P + slot,
                  st + L::K_CHUNKS * 16 + (j * NW + wave) * 1024);
      }
    }
  };
  auto produce = [&](int limit) {
    while (issued < limit && p_item >= 0) {
      issue_tile(p_tile, issued % NSTAGE);
      ++issued;
      if (++p_tile == p_end) {
        if (p_item == cur && nxt >= 0 && nxt < n_items)
          p_set(nxt);
        else
          p_item = -1;  // resumes once the consumer knows the item after this one
      }
    }
  };
  // Workgroup barrier that leaves the newest `pending` issued tiles' loads
  // in flight: this wave's LDS operations and older tile loads complete
  // first.  (__syncthreads would wait for every outstanding global load,
  // the prefetched tiles included.)  Other vector memory operations that
  // are still outstanding only make the wait longer, never shorter, since
  // loads complete in issue order.
  auto sync_tiles = [&](int pending) {
    if (pending >= 2)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOADS_PER_TILE) : "memory");
    else if (pending == 1)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };

  produce(2);
  sync_tiles(issued - 1);

  const int key_a0 = st_row_key(col);  // K row this lane feeds to block 0 (block 1: +32)
  const int vrow_swz = L::v_swz(col);  // V^T rows db*32 + col share it

  while (true) {
    const PrefillItem it = sload(a.items + cur);
    const SeqDesc sd = sload(a.seqs + it.seq);
    const SegDesc sg = sload(a.segs + it.seq * a.num_kv_heads + it.kv_head);
    const int h = it.kv_head * G + (r - pos_off * G);
    const int t0 = it.qtile * rows;
    const int t_last = min(t0 + rows, sd.q_len) - 1;  // last valid query of the tile
    const int t = t0 + pos_off;
    const bool valid = pos_off < rows && t < sd.q_len;
    const int base = sd.kv_len - sd.q_len;
    const int p = base + min(t, t_last);  // invalid columns mimic the last valid row
    const int W = sg.window;
    const int vis_lo = W > 0 ? p - W + 1 : 0;
    const int p_wmin = base + min(t0 + (wave * 32) / G, t_last);
    const int p_wmax = base + min(t0 + (wave * 32 + 31) / G, t_last);

    // Q^T operand, held in registers for the whole item.
    bf16x8 qv[NKK];
    {
      // Loads are unconditional (an invalid row reads the tile's last valid
      // row and is zeroed afterwards), so they are in flight together.
      const uint16_t *qrow = a.q + (static_cast<size_t>(sd.q_start + min(t, t_last)) * a.num_q_heads + h) * D;
      if (sg.rope_off < 0) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 x = ld16(qrow + kk * 16 + half * 8);
          qv[kk] = as_bf16x8(valid ? x : z);
        }
      } else {
        relocate_row<D, NKK>(qv, qrow, 16, half * 8, valid, a.rope.tables + sg.rope_off, s_rope[wave], a.rope);
      }
      // Wait for Q here, once per item; the tile loop then carries no wait
      // on it (the compiler cannot prove the load done inside the loop and
      // would drain every prefetched tile before each product).
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qv[kk]));
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m = kNegInf;  // running (lazy) max of raw scores of this column
    float l = 0.f;      // this lane's share of the running sum

    // One 64-key tile: S^T = K Q^T, (mask), lazy online softmax, O^T += V^T P^T.
    auto process = [&](const char *st, int k0, auto mask_tag) {
      constexpr bool MASK = decltype(mask_tag)::value;
      f32x16 s0 = f32x16{}, s1 = f32x16{};
      // K operands stream two k-steps ahead of the products (scheduling
      // fences keep the compiler from loading all of them up front).
      bf16x8 kr[NKK][2];
      auto kread = [&](int kk) {
        const int c = (2 * kk + half) ^ L::k_swz(key_a0);
        kr[kk][0] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + (key_a0 * L::KCPR + c) * 16));
        kr[kk][1] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + ((key_a0 + 32) * L::KCPR + c) * 16));
      };
      kread(0);
      kread(1);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kk][0], qv[kk], s0, 0, 0, 0);
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kk][1], qv[kk], s1, 0, 0, 0);
        if (kk + 2 < NKK) kread(kk + 2);
      }
      // V^T operands of the first 32 keys, read now so that their latency
      // is hidden behind the softmax.
      bf16x8 vpre[2][NDB];
#pragma unroll
      for (int sh = 0; sh < 2; ++sh)
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          vpre[sh][db] = as_bf16x8(*reinterpret_cast<const u32x4 *>(
              st + ((L::K_CHUNKS + (db * 32 + col) * 8) + ((sh * 2 + half) ^ vrow_swz)) * 16));
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (MASK) {
        // key = k0 + 16 (v/8) + 8 half + v%8 (+32 for block 1); visible iff
        // vis_lo <= key <= p, tested as one unsigned range compare.
        const unsigned lo_rel = static_cast<unsigned>(vis_lo - k0 - 8 * half);
        const unsigned span = static_cast<unsigned>(p - vis_lo);
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int off = ((v >> 3) << 4) + (v & 7);
          if (static_cast<unsigned>(off) - lo_rel > span) s0[v] = kNegInf;
          if (static_cast<unsigned>(off + 32) - lo_rel > span) s1[v] = kNegInf;
        }
      }
      float mx = max32(s0, s1);
      {
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
        mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
      }
      // Lazy running max (the lane pair of a column takes the same decision).
      const bool bump = mx * a.scale_log2 > m * a.scale_log2 + kRescaleLog2;
      const float m_new = bump ? mx : m;
      const float msc = m_new == kNegInf ? 0.f : m_new * a.scale_log2;
      // Rare after the first tiles: a scalar branch on the wave's ballot.
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(bump) != 0, 0)) {
        const float alpha = bump ? fast_exp2(m * a.scale_log2 - msc) : 1.f;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      }
      m = m_new;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s0[v] = fast_exp2(fmaf(s0[v], a.scale_log2, -msc));
        s1[v] = fast_exp2(fmaf(s1[v], a.scale_log2, -msc));
      }
      l += sum32(s0, s1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const f32x16 &sv = kb ? s1 : s0;
          const bf16x8 pb = pack8_bf16(sv[8 * s + 0], sv[8 * s + 1], sv[8 * s + 2], sv[8 * s + 3], sv[8 * s + 4],
                                       sv[8 * s + 5], sv[8 * s + 6], sv[8 * s + 7]);
          const int c = (kb * 4 + s * 2 + half) ^ vrow_swz;
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 va = kb == 0 ? vpre[s][db] :
                as_bf16x8(*reinterpret_cast<const u32x4 *>(st + ((L::K_CHUNKS + (db * 32 + col) * 8) + c) * 16));
            oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
          }
        }
      }
    };

    // Tiles of this item.  The wait before each barrier leaves only the
    // loads issued after the next tile pending.
    const int fetch_tile = max(it.tile_begin, it.tile_end - 3);
    for (int tile = it.tile_begin; tile < it.tile_end; ++tile) {
      if (tile == fetch_tile && tid == 0) s_next[fslot] = atomicAdd(a.counter, 1);
      if (issued <= consumed) {  // the producer fell behind (short items): load this tile now
        produce(consumed + 1);
        sync_tiles(issued - consumed - 1);
      }
      produce(consumed + 3);
      const char *st = smem + (consumed % NSTAGE) * L::STAGE_BYTES;
      const int k0 = tile * kTileKeys;
      const bool empty = k0 > p_wmax || (W > 0 && k0 + kTileKeys - 1 < p_wmin - W + 1);
      const bool full = k0 + kTileKeys - 1 <= p_wmin && (W == 0 || k0 >= p_wmax - W + 1);
      if (!empty) {
        if (full)
          process(st, k0, std::integral_constant<bool, false>{});
        else
          process(st, k0, std::integral_constant<bool, true>{});
      }
      sync_tiles(issued - consumed - 2);
      ++consumed;
      if (tile == fetch_tile) {  // the index fetched in this iteration is visible after its barrier
        nxt = __builtin_amdgcn_readfirstlane(s_next[fslot]);
        fslot ^= 1;
        if (p_item < 0 && nxt < n_items) p_set(nxt);
      }
    }

    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_val = l_tot > 0.f ? m * a.scale + logf(l_tot) : kNegInf;
    if (it.part < 0) {
      // A lane holds 4-channel groups i of its row (channels db*32 + 8 i +
      // 4 half ..); one swap with the partner lane gives each lane 8
      // contiguous channels: lanes 0-31 the groups of even i, 32-63 odd i.
      u32x4 w[NDB][2];
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int ip = 0; ip < 2; ++ip) {
          const f32x16 &ac = oacc[db];
          const u32x2 p0 = pack4_bf16(ac[8 * ip] * inv, ac[8 * ip + 1] * inv, ac[8 * ip + 2] * inv, ac[8 * ip + 3] * inv);
          const u32x2 p1 =
              pack4_bf16(ac[8 * ip + 4] * inv, ac[8 * ip + 5] * inv, ac[8 * ip + 6] * inv, ac[8 * ip + 7] * inv);
#pragma unroll
          for (int k = 0; k < 2; ++k) {
            // lanes 32-63 of the first operand trade with lanes 0-31 of the second
            const auto sw = __builtin_amdgcn_permlane32_swap(p0[k], p1[k], false, false);
            w[db][ip][k] = sw[0];
            w[db][ip][2 + k] = sw[1];
          }
        }
      }
      if (valid) {
        uint16_t *orow = a.o + (static_cast<size_t>(sd.q_start + t) * a.num_q_heads + h) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int ip = 0; ip < 2; ++ip) *reinterpret_cast<u32x4 *>(orow + db * 32 + ip * 16 + half * 8) = w[db][ip];
        if (half == 0 && a.lse) a.lse[static_cast<size_t>(sd.q_start + t) * a.num_q_heads + h] = lse_val;
      }
    } else {
      float *prow = a.part_o + (static_cast<size_t>(it.part) * kPrefillRows + r) * D;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int d0 = db * 32 + i * 8 + half * 4;
          f32x4 x = {oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                     oacc[db][4 * i + 3] * inv};
          *reinterpret_cast<f32x4 *>(prow + d0) = x;
        }
      }
      if (half == 0) a.part_lse[static_cast<size_t>(it.part) * kPrefillRows + r] = lse_val;
    }

    // Next item.  Its index was fetched during the previous item; fetch the
    // one after it now (read after the first tile's barrier).
    if (nxt >= n_items) break;
    cur = nxt;
    nxt = -1;
  }
}

// ===========================================================================
// Prefill, wide variant: 4 waves of 64 rows each (one wave per SIMD), so
// that every K and V^T operand read from LDS feeds two products (one per
// 32-row column block) instead of one.  Each 64-key tile is taken in two
// 32-key steps, software pipelined within the wave: while the products S^T
// = K Q^T of step j+1 run, the wave turns step j's scores into bf16
// probabilities, and while O^T += V^T P^T of step j runs, it masks and
// takes the row maxima of step j+1.  The softmax's vector work thus
// overlaps the same wave's matrix work.
//
// The QK products are issued as inline asm so that their accumulators (the
// scores, read by vector code) stay in ordinary VGPRs; the compiler's own
// PV products then keep the O^T accumulators in AGPRs, and the wave fits its
// registers: 64 (Q) + 2 x 32 (scores of two steps) + 16 (probabilities) +
// operands in VGPRs, 128 accumulators in AGPRs.  The asm products start
// from a zero accumulator or chain on the same registers (which the
// hardware orders), and their results are read by vector code only after
// mfma_guard(), which spaces the read from the last product.
//
// Stage s of a four-stage LDS ring holds one tile's K and V^T: tiles i+2
// and i+3 load while tile i is read (and tile i+1's first half of K, for
// the pipelined step).  Work items, the queue, the split partials and the
// output layout are those of prefill_kernel.
// ===========================================================================

// Accumulator d = A B (first k-step) or d += A B, for 32x32x16 bf16, with
// B (the query operand) read straight from AGPRs, where it stays for the
// whole work item.
__device__ __forceinline__ void mfma_qk_first(f32x16 &d, const bf16x8 &a, const bf16x8 &b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_qk(f32x16 &d, const bf16x8 &a, const bf16x8 &b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
// Results of the asm products are read by vector instructions only after
// this (24 wait states cover the 32x32x16 product's write-back; the
// compiler does not know the asm's latency and would not insert them).
__device__ __forceinline__ void mfma_guard(f32x16 &x, f32x16 &y) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(x), "+v"(y));
}

__device__ __forceinline__ float max16(const f32x16 &x) {
  const float a = fmaxf(fmaxf(x[0], x[1]), x[2]), b = fmaxf(fmaxf(x[3], x[4]), x[5]);
  const float c = fmaxf(fmaxf(x[6], x[7]), x[8]), d = fmaxf(fmaxf(x[9], x[10]), x[11]);
  const float e = fmaxf(fmaxf(x[12], x[13]), x[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), x[15]));
}

template <int D, int P>
__global__ __launch_bounds__(kPrefillWideThreads, 1) void prefill_wide_kernel(PrefillArgs a) {
  using L = PrefillLds<D>;
  constexpr int NKK = D / 16;  // k-steps of the QK product
  constexpr int NDB = D / 32;  // 32-channel blocks of O^T
  constexpr int NW = kPrefillWideThreads / 64;
  constexpr int K_INSTR = L::K_CHUNKS / kPrefillWideThreads;  // direct loads per lane per tile (K)
  constexpr int V_INSTR = L::V_CHUNKS / kPrefillWideThreads;  // (V^T)
  constexpr int NSTAGE = 4;
  constexpr int LOADS_PER_TILE = K_INSTR + V_INSTR;
  static_assert(kPrefillRows == 64 * NW, "two 32-row column blocks per wave");
  static_assert(K_INSTR >= 1 && V_INSTR >= 1, "tile smaller than one load per lane");
  static_assert(8 % NKK == 0 || NKK % 8 == 0, "softmax slices per k-step");
  __shared__ __attribute__((aligned(16))) uint4 smem4[NSTAGE * L::STAGE_BYTES / 16];
  __shared__ int s_next[2];
  __shared__ __attribute__((aligned(16))) float s_rope[NW][2 * D];
  char *smem = reinterpret_cast<char *>(smem4);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int G = a.group;
  const int rows = a.rows_per_tile;
  const int n_items = a.n_items;

  if (tid == 0) s_next[0] = atomicAdd(a.counter, 1);
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(s_next[0]);
  if (cur >= n_items) return;
  int nxt = -1;
  int fslot = 1;

  // Producer: K/V tile loads run ahead of the consumer along this
  // workgroup's sequence of tiles, across item boundaries.
  int p_item = -1, p_tile = 0, p_end = 0;
  SegDesc psg;
  auto p_set = [&](int idx) {
    const PrefillItem pi_ = sload(a.items + idx);
    p_item = idx;
    p_tile = pi_.tile_begin;
    p_end = pi_.tile_end;
    psg = sload(a.segs + pi_.seq * a.num_kv_heads + pi_.kv_head);
  };
  p_set(cur);
  int issued = 0;  // tiles issued so far (index in this workgroup's tile sequence)
  int ready = 0;   // tiles known to have landed in LDS and passed a barrier
  auto issue_tile = [&](int tile, int stage) {
    const int k0 = tile * kTileKeys;
    const int last_page = psg.n_pages - 1;
    char *st = smem + stage * L::STAGE_BYTES;
    constexpr int NP = kTileKeys / P;
    int pid[NP];
    const int pg0 = (k0 - psg.first_token) / P;
#pragma unroll
    for (int i = 0; i < NP; ++i) pid[i] = sload(a.page_ids + psg.page_off + min(max(pg0 + i, 0), last_page));
    auto page_of = [&](int key_in_tile, int *slot) {
      const int rel = k0 + key_in_tile - psg.first_token;
      *slot = rel >= 0 && rel / P <= last_page ? key_in_tile % P : 0;
      int page = pid[0];
#pragma unroll
      for (int i = 1; i < NP; ++i)
        if (key_in_tile / P == i) page = pid[i];
      return page;
    };
#pragma unroll
    for (int j = 0; j < K_INSTR; ++j) {
      const int c = (j * NW + wave) * 64 + lane;
      const int row = c / L::KCPR;
      const int logical = (c % L::KCPR) ^ L::k_swz(row);
      const uint16_t *src;
      if constexpr (P == kTileKeys) {
        src = a.k_pool + static_cast<size_t>(pid[0]) * (P * D) + row * D + logical * 8;
      } else {
        int slot;
        const int page = page_of(row, &slot);
        src = a.k_pool + (static_cast<size_t>(page) * P + slot) * D + logical * 8;
      }
      lds_dma16(src, st + (j * NW + wave) * 1024);
    }
#pragma unroll
    for (int j = 0; j < V_INSTR; ++j) {
      const int c = (j * NW + wave) * 64 + lane;
      const int d = c / 8;
      const int logical = (c % 8) ^ L::v_swz(d);
      const uint16_t *src;
      if constexpr (P == kTileKeys) {
        src = a.v_pool + static_cast<size_t>(pid[0]) * (P * D) + d * P + logical * 8;
      } else {
        int slot;
        const int page = page_of(logical * 8, &slot);
        src = a.v_pool + static_cast<size_t>(page) * (P * D) + d * P + slot;
      }
      lds_dma16(src, st + L::K_CHUNKS * 16 + (j * NW + wave) * 1024);
    }
  };
  auto produce = [&](int limit) {
    while (issued < limit && p_item >= 0) {
      issue_tile(p_tile, issued % NSTAGE);
      ++issued;
      if (++p_tile == p_end) {
        if (p_item == cur && nxt >= 0 && nxt < n_items)
          p_set(nxt);
        else
          p_item = -1;
      }
    }
  };
  // Barrier that leaves the newest `pending` issued tiles' loads in flight
  // (see prefill_kernel); every older tile is then ready.
  auto sync_tiles = [&](int pending) {
    if (pending >= 2) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOADS_PER_TILE) : "memory");
      ready = issued - 2;
    } else if (pending == 1) {
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
      ready = issued - 1;
    } else {
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      ready = issued;
    }
  };
  // Tile g of the sequence must be ready before it is read: when the
  // producer fell behind (short items), issue it now and wait for it.
  auto ensure_ready = [&](int g) {
    if (ready <= g) {
      produce(g + 1);
      sync_tiles(0);
    }
  };

  produce(3);
  sync_tiles(issued - 1);
  int consumed = 0;  // tiles of the sequence fully computed

  const int key_a0 = st_row_key(col);
  const int vrow_swz = L::v_swz(col);

  while (true) {
    const PrefillItem it = sload(a.items + cur);
    const SeqDesc sd = sload(a.seqs + it.seq);
    const SegDesc sg = sload(a.segs + it.seq * a.num_kv_heads + it.kv_head);
    const int t0 = it.qtile * rows;
    const int t_last = min(t0 + rows, sd.q_len) - 1;
    const int base = sd.kv_len - sd.q_len;
    const int W = sg.window;
    const int p_wmin = base + min(t0 + (wave * 64) / G, t_last);
    const int p_wmax = base + min(t0 + (wave * 64 + 63) / G, t_last);
    // The two rows of this lane: column blocks c = 0, 1.
    int hh[2], tt[2], pp[2], lo[2];
    bool valid[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int r = wave * 64 + 32 * c + col;
      const int po = r / G;
      hh[c] = it.kv_head * G + (r - po * G);
      tt[c] = t0 + po;
      valid[c] = po < rows && tt[c] < sd.q_len;
      pp[c] = base + min(tt[c], t_last);
      lo[c] = W > 0 ? pp[c] - W + 1 : 0;
    }

    bf16x8 qv[2][NKK];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint16_t *qrow =
          a.q + (static_cast<size_t>(sd.q_start + min(tt[c], t_last)) * a.num_q_heads + hh[c]) * D;
      if (sg.rope_off < 0) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 x = ld16(qrow + kk * 16 + half * 8);
          qv[c][kk] = as_bf16x8(valid[c] ? x : z);
        }
      } else {
        relocate_row<D, NKK>(qv[c], qrow, 16, half * 8, valid[c], a.rope.tables + sg.rope_off, s_rope[wave], a.rope);
      }
    }
    // Q is waited for here, once per item, and moved to AGPRs; the two wait
    // states after the last of those writes precede its first read by an
    // asm product.
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+a"(qv[c][kk]));
    asm volatile("s_nop 1" ::: "memory");

    f32x16 oacc[2][NDB];
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[c][db] = f32x16{};
    float m[2] = {kNegInf, kNegInf};
    float l[2] = {0.f, 0.f};
    float msc[2] = {0.f, 0.f};

    auto stage_of = [&](int g) { return smem + (g % NSTAGE) * L::STAGE_BYTES; };
    // K operand of k-step kk for the 32-key half h of a tile; V^T operand of
    // 16-key step ks (0..3) of a tile, channel block db.
    auto k_frag = [&](const char *st, int kk, int h) {
      const int c = (2 * kk + half) ^ L::k_swz(key_a0);
      return as_bf16x8(*reinterpret_cast<const u32x4 *>(st + ((key_a0 + 32 * h) * L::KCPR + c) * 16));
    };
    auto v_frag = [&](const char *st, int ks, int db) {
      const int c = ((ks >> 1) * 4 + (ks & 1) * 2 + half) ^ vrow_swz;
      return as_bf16x8(*reinterpret_cast<const u32x4 *>(st + ((L::K_CHUNKS + (db * 32 + col) * 8) + c) * 16));
    };
    // A 32-key step is fully visible to every row of this wave when:
    auto step_full = [&](int k0) { return k0 + 31 <= p_wmin && (W == 0 || k0 >= p_wmax - W + 1); };

    f32x16 sc[2];          // scores of the current 32-key step (c = 0, 1)
    bf16x8 pkA[2][2], pkB[2][2];  // probabilities of even / odd steps: [c][16-key half]
    float alpha[2] = {1.f, 1.f};
    bool rescale = false;  // O^T waits for its rescale until the previous step's PV is in

    // Mask (edge steps), row maxima across the lane pair and the lazy
    // rescale decision: the running max moves only when a step's max exceeds
    // it by more than 2^8.  Rows with no visible key yet hold O = 0 and l = 0
    // and need no rescale.  l is rescaled at once; O^T after the previous
    // step's products are accumulated (it must include them).
    auto head = [&](int k0, bool mask) {
      bool bump[2], need[2];
      float m_new[2];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        if (mask) {
          const unsigned lo_rel = static_cast<unsigned>(lo[c] - k0 - 8 * half);
          const unsigned span = static_cast<unsigned>(pp[c] - lo[c]);
#pragma unroll
          for (int v = 0; v < 16; ++v) {
            const int off = ((v >> 3) << 4) + (v & 7);
            if (static_cast<unsigned>(off) - lo_rel > span) sc[c][v] = kNegInf;
          }
        }
        float x = max16(sc[c]);
        const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
        x = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
        bump[c] = x * a.scale_log2 > m[c] * a.scale_log2 + kRescaleLog2;
        need[c] = bump[c] && m[c] != kNegInf;
        m_new[c] = bump[c] ? x : m[c];
      }
      rescale = __builtin_amdgcn_ballot_w64(need[0] || need[1]) != 0;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float ms = m_new[c] == kNegInf ? 0.f : m_new[c] * a.scale_log2;
        alpha[c] = need[c] ? fast_exp2(m[c] * a.scale_log2 - ms) : 1.f;
        l[c] *= alpha[c];
        m[c] = m_new[c];
        msc[c] = ms;
      }
    };
    auto apply_rescale = [&]() {
      if (__builtin_expect(rescale, 0)) {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[c][db] *= alpha[c];
      }
    };
    // Probabilities of values v0 .. v0+nv-1 of the current scores into pk.
    auto body = [&](bf16x8 (&pk)[2][2], int c, int v0, int nv) {
#pragma unroll
      for (int u = 0; u < nv; ++u) {
        sc[c][v0 + u] = fast_exp2(fmaf(sc[c][v0 + u], a.scale_log2, -msc[c]));
        l[c] += sc[c][v0 + u];
      }
      // pack each group of 8 whose last value this slice computed
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        if (v0 <= 8 * w + 7 && 8 * w + 7 < v0 + nv) {
          const f32x16 &x = sc[c];
          pk[c][w] = pack8_bf16(x[8 * w], x[8 * w + 1], x[8 * w + 2], x[8 * w + 3], x[8 * w + 4], x[8 * w + 5],
                                x[8 * w + 6], x[8 * w + 7]);
        }
      }
    };
    // S^T of half h of the tile in st into sc (K operands one k-step ahead).
    auto qk_step = [&](const char *st, int h) {
      bf16x8 kf = k_frag(st, 0, h);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        __builtin_amdgcn_sched_barrier(0);
        const bf16x8 kn = kk + 1 < NKK ? k_frag(st, kk + 1, h) : kf;
        if (kk == 0) {
          mfma_qk_first(sc[0], kf, qv[0][0]);
          mfma_qk_first(sc[1], kf, qv[1][0]);
        } else {
          mfma_qk(sc[0], kf, qv[0][kk]);
          mfma_qk(sc[1], kf, qv[1][kk]);
        }
        kf = kn;
      }
      __builtin_amdgcn_sched_barrier(0);
      mfma_guard(sc[0], sc[1]);
    };
    // O^T += V^T P^T for half h of the tile in st with probabilities pk_prev,
    // and after each product pair a slice of the current step's body into
    // pk_cur (pk_prev == nullptr: the body alone).
    auto pv_body = [&](const char *st, int h, bf16x8 (*pk_prev)[2][2], bf16x8 (&pk_cur)[2][2]) {
      constexpr int NG = 2 * NDB;   // product pairs
      constexpr int VPG = 32 / NG;  // body values per pair
      if (!pk_prev) {
#pragma unroll
        for (int c = 0; c < 2; ++c) body(pk_cur, c, 0, 16);
        return;
      }
      bf16x8 vf = v_frag(st, 2 * h, 0);
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        const int ks = g / NDB, db = g % NDB;
        const bf16x8 vn = g + 1 < NG ? v_frag(st, 2 * h + (g + 1) / NDB, (g + 1) % NDB) : vf;
#pragma unroll
        for (int c = 0; c < 2; ++c)
          oacc[c][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, (*pk_prev)[c][ks], oacc[c][db], 0, 0, 0);
        const int j0 = g * VPG;
        body(pk_cur, j0 / 16, j0 % 16, VPG);
        vf = vn;
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    // PV of the last step alone.
    auto pv_last = [&](const char *st, int h, bf16x8 (&pk)[2][2]) {
      bf16x8 vf = v_frag(st, 2 * h, 0);
#pragma unroll
      for (int g = 0; g < 2 * NDB; ++g) {
        __builtin_amdgcn_sched_barrier(0);
        const int ks = g / NDB, db = g % NDB;
        const bf16x8 vn = g + 1 < 2 * NDB ? v_frag(st, 2 * h + (g + 1) / NDB, (g + 1) % NDB) : vf;
#pragma unroll
        for (int c = 0; c < 2; ++c)
          oacc[c][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pk[c][ks], oacc[c][db], 0, 0, 0);
        vf = vn;
      }
    };

    const int n_tiles = it.tile_end - it.tile_begin;
    const int fetch_t = max(0, n_tiles - 3);  // tile whose closing barrier publishes the next item's index
    const int g0 = consumed;
    const int kb0 = it.tile_begin * kTileKeys;

    // Tile t's bookkeeping around its two steps: the producer before, the
    // barrier (and the next item's index) after.
    auto tile_begin = [&](int t) {
      if (t == fetch_t && tid == 0) s_next[fslot] = atomicAdd(a.counter, 1);
      produce(g0 + t + 3);
      ensure_ready(g0 + t);
    };
    auto tile_end = [&](int t) {
      sync_tiles(issued - (g0 + t) - 2);
      if (t == fetch_t) {
        nxt = __builtin_amdgcn_readfirstlane(s_next[fslot]);
        fslot ^= 1;
        if (p_item < 0 && nxt < n_items) p_set(nxt);
      }
    };
    // Tile 0: its first step has no previous products (and O^T = 0 needs no
    // rescale).
    {
      tile_begin(0);
      const char *st = stage_of(g0);
      qk_step(st, 0);
      head(kb0, !step_full(kb0));
      pv_body(st, 1, nullptr, pkA);
      qk_step(st, 1);
      head(kb0 + 32, !step_full(kb0 + 32));
      pv_body(st, 0, &pkA, pkB);
      apply_rescale();
      tile_end(0);
    }
    for (int t = 1; t < n_tiles; ++t) {
      tile_begin(t);
      const char *st = stage_of(g0 + t);
      const int k0 = kb0 + t * kTileKeys;
      // step 2t: half 0 of tile t; the products of step 2t-1 (half 1 of the
      // previous tile) run under its softmax body
      qk_step(st, 0);
      head(k0, !step_full(k0));
      pv_body(stage_of(g0 + t - 1), 1, &pkB, pkA);
      apply_rescale();
      // step 2t+1: half 1 of tile t, with the products of step 2t
      qk_step(st, 1);
      head(k0 + 32, !step_full(k0 + 32));
      pv_body(st, 0, &pkA, pkB);
      apply_rescale();
      tile_end(t);
    }
    pv_last(stage_of(g0 + n_tiles - 1), 1, pkB);
    consumed = g0 + n_tiles;

#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const float l_tot = l[c] + __shfl_xor(l[c], 32);
      const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
      const float lse_val = l_tot > 0.f ? m[c] * a.scale + logf(l_tot) : kNegInf;
      const int r = wave * 64 + 32 * c + col;
      if (it.part < 0) {
        u32x4 w[NDB][2];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int ip = 0; ip < 2; ++ip) {
            const f32x16 &ac = oacc[c][db];
            const u32x2 p0 =
                pack4_bf16(ac[8 * ip] * inv, ac[8 * ip + 1] * inv, ac[8 * ip + 2] * inv, ac[8 * ip + 3] * inv);
            const u32x2 p1 =
                pack4_bf16(ac[8 * ip + 4] * inv, ac[8 * ip + 5] * inv, ac[8 * ip + 6] * inv, ac[8 * ip + 7] * inv);
#pragma unroll
            for (int k = 0; k < 2; ++k) {
              const auto sw = __builtin_amdgcn_permlane32_swap(p0[k], p1[k], false, false);
              w[db][ip][k] = sw[0];
              w[db][ip][2 + k] = sw[1];
            }
          }
        }
        if (valid[c]) {
          uint16_t *orow = a.o + (static_cast<size_t>(sd.q_start + tt[c]) * a.num_q_heads + hh[c]) * D;
#pragma unroll
          for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int ip = 0; ip < 2; ++ip)
              *reinterpret_cast<u32x4 *>(orow + db * 32 + ip * 16 + half * 8) = w[db][ip];
          if (half == 0 && a.lse) a.lse[static_cast<size_t>(sd.q_start + tt[c]) * a.num_q_heads + hh[c]] = lse_val;
        }
      } else {
        float *prow = a.part_o + (static_cast<size_t>(it.part) * kPrefillRows + r) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int d0 = db * 32 + i * 8 + half * 4;
            f32x4 x = {oacc[c][db][4 * i] * inv, oacc[c][db][4 * i + 1] * inv, oacc[c][db][4 * i + 2] * inv,
                       oacc[c][db][4 * i + 3] * inv};
            *reinterpret_cast<f32x4 *>(prow + d0) = x;
          }
        }
        if (half == 0) a.part_lse[static_cast<size_t>(it.part) * kPrefillRows + r] = lse_val;
      }
    }

    if (nxt >= n_items) break;
    cur = nxt;
    nxt = -1;
  }
}

// ===========================================================================
// Attention-mass token scores ("attention as a router" for the sparse FFN:
// "Xiaohongshu Open-Sources RedKnot" page, "What Happened" item 2; "RedKnot:
// Head-Aware KV Reuse and SegPagedAttention" page, "The Three Core
// Mechanisms in Detail", second mechanism).  A second pass over the prefill's
// work: with the rows' final LSE known, key j receives sum over rows (t, h)
// of exp(scale q.k_j - lse).  The product is taken as S = Q K^T (operands of
// the prefill's S^T swapped), so a lane holds one key column and 16 query
// rows and the sum over queries is in-lane plus one lane-pair swap.  The 8
// waves' per-tile key sums meet in a double-buffered LDS exchange that rides
// on the K pipeline's per-tile barrier; one wave writes the tile's 64 sums
// as a partial row.  Partial rows are added by score_reduce_kernel in a
// fixed order, so the scores do not depend on the work order.
// ===========================================================================

template <int D, int P>
__global__ __launch_bounds__(kPrefillThreads, 2) void score_kernel(ScoreArgs a) {
  using L = PrefillLds<D>;
  constexpr int NKK = D / 16;
  constexpr int NW = kPrefillThreads / 64;
  constexpr int K_INSTR = L::K_CHUNKS / kPrefillThreads;
  constexpr int NSTAGE = 3;
  constexpr int KSTAGE = L::K_CHUNKS * 16;  // bytes of one K tile
  constexpr float kLog2e = 1.4426950408889634f;
  static_assert(kPrefillRows == 32 * NW && K_INSTR >= 1, "tile layout");
  __shared__ __attribute__((aligned(16))) uint4 smem4[NSTAGE * KSTAGE / 16];
  __shared__ float sx[2][NW][kTileKeys];
  __shared__ __attribute__((aligned(16))) float s_rope[NW][2 * D];  // per-wave relocation table
  char *smem = reinterpret_cast<char *>(smem4);

  const PrefillItem it = sload(a.items + blockIdx.x);
  const SeqDesc sd = sload(a.seqs + it.seq);
  const SegDesc sg = sload(a.segs + it.seq * a.num_kv_heads + it.kv_head);
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int G = a.group;
  const int rows = a.rows_per_tile;
  const int t0 = it.qtile * rows;
  const int t_last = min(t0 + rows, sd.q_len) - 1;
  const int base = sd.kv_len - sd.q_len;
  const int W = sg.window;
  const int p_wmin = base + min(t0 + (wave * 32) / G, t_last);
  const int p_wmax = base + min(t0 + (wave * 32 + 31) / G, t_last);

  // Q operand (A of S = Q K^T): this lane supplies query row wave*32 + col.
  bf16x8 qv[NKK];
  {
    const int r = wave * 32 + col;
    const int po = r / G;
    const int h = it.kv_head * G + (r - po * G);
    const int t = t0 + po;
    const bool valid = po < rows && t < sd.q_len;
    // Loads are unconditional (an invalid row reads the tile's last valid
    // row and is zeroed afterwards), so they are in flight together.
    const uint16_t *qrow = a.q + (static_cast<size_t>(sd.q_start + min(t, t_last)) * a.num_q_heads + h) * D;
    if (sg.rope_off < 0) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        const u32x4 z = {0u, 0u, 0u, 0u};
        const u32x4 x = ld16(qrow + kk * 16 + half * 8);
        qv[kk] = as_bf16x8(valid ? x : z);
      }
    } else {
      relocate_row<D, NKK>(qv, qrow, 16, half * 8, valid, a.rope.tables + sg.rope_off, s_rope[wave], a.rope);
    }
  }
  // The rows of S this lane holds: register v is row 8 (v/4) + 4 half + v%4
  // of the wave.  Rows past the chunk get lse = +inf, hence probability 0.
  // Each lane loads the LSE of its own row (one coalesced load: an invalid
  // row reads the tile's last valid row and gets +inf); lane v's rows are
  // then taken from the lanes that loaded them.
  float lse_own;
  {
    const int r = wave * 32 + col;
    const int po = r / G;
    const int t = t0 + po;
    const bool valid = po < rows && t < sd.q_len;
    const float raw = a.lse[static_cast<size_t>(sd.q_start + min(t, t_last)) * a.num_q_heads + it.kv_head * G +
                            (r - po * G)];
    lse_own = valid ? raw * kLog2e : __builtin_inff();
  }
  float lse2[16];
  int prow[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int rw = 8 * (v >> 2) + 4 * half + (v & 3);  // row within the wave
    const int po = (wave * 32 + rw) / G;
    const int t = t0 + po;
    lse2[v] = __shfl(lse_own, rw);
    prow[v] = base + min(t, t_last);
  }
  // Wait for Q and the LSE values once, here; inside the tile loop the
  // compiler would otherwise wait for every outstanding load (the
  // prefetched tiles included) before their first use in each tile.
#pragma unroll
  for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qv[kk]));
#pragma unroll
  for (int v = 0; v < 16; ++v) asm volatile("" : "+v"(lse2[v]));

  const int last_page = sg.n_pages - 1;
  auto issue_tile = [&](int tile, int stage) {
    const int k0 = tile * kTileKeys;
    char *st = smem + stage * KSTAGE;
    // Page ids of the tile's NP whole pages by scalar loads (as in the
    // prefill); keys outside the stored pages read slot 0 of the nearest.
    constexpr int NP = kTileKeys / P;
    int pid[NP];
    const int pg0 = (k0 - sg.first_token) / P;
#pragma unroll
    for (int i = 0; i < NP; ++i) pid[i] = sload(a.page_ids + sg.page_off + min(max(pg0 + i, 0), last_page));
#pragma unroll
    for (int j = 0; j < K_INSTR; ++j) {
      const int c = (j * NW + wave) * 64 + lane;
      const int row = c / L::KCPR;
      const int logical = (c % L::KCPR) ^ L::k_swz(row);
      if constexpr (P == kTileKeys) {
        // one page per tile: a scalar page base and a 32-bit lane offset
        lds_dma16_s(a.k_pool + static_cast<size_t>(pid[0]) * (P * D), static_cast<uint32_t>((row * D + logical * 8) * 2),
                    st + (j * NW + wave) * 1024);
      } else {
        const int rel = k0 + row - sg.first_token;
        const int slot = rel >= 0 && rel / P <= last_page ? row % P : 0;
        int page = pid[0];
#pragma unroll
        for (int i = 1; i < NP; ++i)
          if (row / P == i) page = pid[i];
        lds_dma16(a.k_pool + (static_cast<size_t>(page) * P + slot) * D + logical * 8, st + (j * NW + wave) * 1024);
      }
    }
  };

  const int kswz = L::k_swz(col);  // keys col and col + 32 share it
  // Key sums of one tile over this wave's 32 rows: c0 for key k0 + col, c1
  // for key k0 + 32 + col (both lanes of a pair end with the full sums).
  auto process = [&](const char *st, int k0, auto mask_tag, float &c0, float &c1) {
    constexpr bool MASK = decltype(mask_tag)::value;
    f32x16 s0 = f32x16{}, s1 = f32x16{};
    // K operands stream two k-steps ahead of the products (scheduling
    // fences keep the compiler from loading all of them up front).
    bf16x8 kr[NKK][2];
    auto kread = [&](int kk) {
      const int c = (2 * kk + half) ^ kswz;
      kr[kk][0] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + (col * L::KCPR + c) * 16));
      kr[kk][1] = as_bf16x8(*reinterpret_cast<const u32x4 *>(st + ((col + 32) * L::KCPR + c) * 16));
    };
    kread(0);
    kread(1);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      __builtin_amdgcn_sched_barrier(0);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qv[kk], kr[kk][0], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qv[kk], kr[kk][1], s1, 0, 0, 0);
      if (kk + 2 < NKK) kread(kk + 2);
    }
    __builtin_amdgcn_sched_barrier(0);
    float e0 = 0.f, e1 = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float x0 = fmaf(s0[v], a.scale_log2, -lse2[v]);
      float x1 = fmaf(s1[v], a.scale_log2, -lse2[v]);
      if constexpr (MASK) {
        const int key0 = k0 + col, key1 = key0 + 32;
        const int lo = W > 0 ? prow[v] - W + 1 : 0;
        if (key0 > prow[v] || key0 < lo) x0 = kNegInf;
        if (key1 > prow[v] || key1 < lo) x1 = kNegInf;
      }
      e0 += fast_exp2(x0);
      e1 += fast_exp2(x1);
    }
    c0 = e0 + __shfl_xor(e0, 32);
    c1 = e1 + __shfl_xor(e1, 32);
  };
  // Tile i's sums of all waves are in sx[i % 2] after the barrier ending
  // iteration i; wave i % NW adds them (fixed order) during iteration i + 1.
  auto flush = [&](int i) {
    if (wave == i % NW) {
      float acc = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) acc += sx[i & 1][w][lane];
      a.part[(static_cast<size_t>(it.part) + i) * kTileKeys + lane] = acc;
    }
  };

  constexpr int LOADS_PER_TILE = K_INSTR;
  const int tb = it.tile_begin, te = it.tile_end;
  // Barriers leave the newest tile's loads in flight (see the prefill).
  if (tb < te) issue_tile(tb, 0);
  if (tb + 1 < te) {
    issue_tile(tb + 1, 1);
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  for (int tile = tb; tile < te; ++tile) {
    const int i = tile - tb;
    const bool ahead2 = tile + 2 < te;
    if (ahead2) issue_tile(tile + 2, (i + 2) % NSTAGE);
    if (i > 0) flush(i - 1);
    const char *st = smem + (i % NSTAGE) * KSTAGE;
    const int k0 = tile * kTileKeys;
    const bool empty = k0 > p_wmax || (W > 0 && k0 + kTileKeys - 1 < p_wmin - W + 1);
    const bool full = k0 + kTileKeys - 1 <= p_wmin && (W == 0 || k0 >= p_wmax - W + 1);
    float c0 = 0.f, c1 = 0.f;
    if (!empty) {
      if (full)
        process(st, k0, std::integral_constant<bool, false>{}, c0, c1);
      else
        process(st, k0, std::integral_constant<bool, true>{}, c0, c1);
    }
    sx[i & 1][wave][half * 32 + col] = half ? c1 : c0;
    if (ahead2)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  }
  if (te > tb) flush(te - tb - 1);
}

// Scores of the chunk's keys: one workgroup per 64-key tile, 16 waves.  A
// pass of wave w covers the 64 partial rows part_idx[base .. base + 64) with
// base = begin + 64 w + 1024 j: each lane loads one of the 64 row indices,
// and load u of lane l (u < 16) reads 16 bytes (keys 4 (l % 16) ..) of row
// 4 u + l / 16, with the row index taken from the lane that loaded it.  The
// sums go lane by lane in load order, then over the 4 lanes of one key
// group and over the 16 waves in a fixed tree, so the result is the same on
// every run for the same partial rows in the same order.
constexpr int kReduceWaves = 16;

__global__ __launch_bounds__(64 * kReduceWaves) void score_reduce_kernel(ScoreReduceArgs a) {
  __shared__ f32x4 red[kReduceWaves][kTileKeys / 4];
  const ScoreRow row = sload(a.rows + blockIdx.x);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int sub = lane >> 4, chunk = lane & 15;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int base = row.begin + 64 * w; base < row.end; base += 64 * kReduceWaves) {
    const int idx = a.part_idx[min(base + lane, row.end - 1)];
    f32x4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int pi = __shfl(idx, 4 * u + sub);
      v[u] = *reinterpret_cast<const f32x4 *>(a.part + static_cast<size_t>(pi) * kTileKeys + 4 * chunk);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (base + 4 * u + sub < row.end) acc += v[u];
  }
#pragma unroll
  for (int x = 16; x <= 32; x <<= 1) {
    f32x4 o;
#pragma unroll
    for (int c = 0; c < 4; ++c) o[c] = __shfl_xor(acc[c], x);
    acc += o;
  }
  if (lane < 16) red[w][chunk] = acc;
  __syncthreads();
  if (w == 0) {
    const float *r = reinterpret_cast<const float *>(red);
    float t[kReduceWaves];
#pragma unroll
    for (int i = 0; i < kReduceWaves; ++i) t[i] = r[i * kTileKeys + lane];
#pragma unroll
    for (int h = kReduceWaves / 2; h >= 1; h >>= 1)
#pragma unroll
      for (int i = 0; i < h; ++i) t[i] += t[i + h];
    const SeqDesc sd = sload(a.seqs + row.seq);
    const int key = row.tile * kTileKeys + lane;
    const int kbase = sd.kv_len - sd.q_len;
    if (key >= kbase && key < sd.kv_len) a.scores[sd.q_start + key - kbase] = t[0];
  }
}

// Top-k per sequence by radix select on the score bits (scores are >= 0, so
// their bit patterns order like the values), ties to the lower index; the
// kept indices are written in ascending order.  One workgroup per sequence;
// each thread holds kTopkRun consecutive keys per batch, so one batch of
// loads is in flight per pass rather than one load per 1024 keys.
__device__ __forceinline__ int block_excl_scan(int x, int *s_wave, int *total) {
  // exclusive prefix sum of x over the workgroup, in thread order
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int inc = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int t = __shfl_up(inc, d);
    if (lane >= d) inc += t;
  }
  if (lane == 63) s_wave[wave] = inc;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / 64; ++w) {
    const int c = s_wave[w];
    if (w < wave) off += c;
    tot += c;
  }
  __syncthreads();
  *total = tot;
  return off + inc - x;
}

__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
  constexpr int NWV = kTopkThreads / 64;
  constexpr int R = kTopkRun;
  constexpr int BATCH = kTopkThreads * R;
  static_assert(BATCH < 65536, "per-batch counts are packed in 16 bits");
  __shared__ int hist[NWV][256];  // one histogram per wave
  __shared__ int s_wave[NWV];
  __shared__ int s_pick[3];
  const int b = blockIdx.x;
  const int n = a.cu[b + 1] - a.cu[b];
  const int k = a.k[b];
  const uint32_t *key = reinterpret_cast<const uint32_t *>(a.scores + a.cu[b]);
  int32_t *out = a.out + a.out_off[b];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (k <= 0) return;
  // A sequence of at most BATCH keys is loaded once and kept in registers
  // for every pass; longer ones are read again in each pass.
  const bool one = n <= BATCH;
  uint32_t xk[R];
  if (one) {
    const int j0 = threadIdx.x * R;
#pragma unroll
    for (int r = 0; r < R; ++r) xk[r] = j0 + r < n ? key[j0 + r] : 0u;
  }
  auto load_batch = [&](int base, uint32_t (&x)[R]) {
    const int j0 = base + threadIdx.x * R;
#pragma unroll
    for (int r = 0; r < R; ++r) x[r] = one ? xk[r] : (j0 + r < n ? key[j0 + r] : 0u);
  };
  uint32_t prefix = 0, mask = 0;
  int need = k;  // how many of the keys matching prefix/mask are still to take
  if (k < n) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = threadIdx.x; i < NWV * 256; i += kTopkThreads) (&hist[0][0])[i] = 0;
      __syncthreads();
      for (int base = 0; base < n; base += BATCH) {
        const int j0 = base + threadIdx.x * R;
        uint32_t x[R];
        load_batch(base, x);
        // Runs of equal bins among a thread's keys are added at once (in
        // the first pass most keys share one bin).
        int run_bin = -1, run_len = 0;
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const int bin = j0 + r < n && (x[r] & mask) == prefix ? static_cast<int>((x[r] >> shift) & 255u) : -1;
          if (bin != run_bin) {
            if (run_len > 0) atomicAdd(&hist[wave][run_bin], run_len);
            run_bin = bin;
            run_len = 0;
          }
          if (bin >= 0) ++run_len;
        }
        if (run_len > 0) atomicAdd(&hist[wave][run_bin], run_len);
      }
      __syncthreads();
      // Per-bin totals, then suffix sums (keys with a bin >= b) by a shuffle
      // scan in each of the first four waves; the one bin where the suffix
      // reaches `need` is the k-th key's bin.
      int cnt = 0, sfx = 0;
      if (threadIdx.x < 256) {
#pragma unroll
        for (int w = 0; w < NWV; ++w) cnt += hist[w][threadIdx.x];
        sfx = cnt;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const int t = __shfl_down(sfx, d);
          if (lane + d < 64) sfx += t;
        }
        if (lane == 0) s_wave[wave] = sfx;  // total of this wave's 64 bins
      }
      __syncthreads();
      if (threadIdx.x < 256) {
        for (int w = wave + 1; w < 4; ++w) sfx += s_wave[w];
        const int above = sfx - cnt;  // keys in higher bins
        if (sfx >= need && above < need) {
          s_pick[0] = threadIdx.x;
          s_pick[1] = need - above;
          s_pick[2] = cnt;
        }
      }
      __syncthreads();
      prefix |= static_cast<uint32_t>(s_pick[0]) << shift;
      mask |= 255u << shift;
      need = s_pick[1];
      const bool whole_bin = s_pick[2] == need;  // every key of the bin is kept: no lower digit matters
      __syncthreads();
      if (whole_bin) break;
    }
  }
  // Keep every key whose masked bits exceed prefix and the first `need`
  // keys whose masked bits equal it, in index order (k >= n keeps
  // everything).  After all four passes the mask is the whole key; a pass
  // that kept its whole bin stops early, and then every equal key is kept.  A kept key's output slot is the
  // number of greater keys before it plus min(equal keys before it, need);
  // both counts come from one scan of the packed per-thread counts.
  int gt_seen = 0, eq_seen = 0;
  for (int base = 0; base < n; base += BATCH) {
    const int j0 = base + threadIdx.x * R;
    uint32_t x[R];
    load_batch(base, x);
    int gt_c = 0, eq_c = 0;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool in = j0 + r < n;
      gt_c += in && (k >= n || (x[r] & mask) > prefix);
      eq_c += in && k < n && (x[r] & mask) == prefix;
    }
    int tot;
    const int ex = block_excl_scan(gt_c | (eq_c << 16), s_wave, &tot);
    int g = gt_seen + (ex & 0xffff), e = eq_seen + (ex >> 16);
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const bool in = j0 + r < n;
      if (in && (k >= n || (x[r] & mask) > prefix)) {
        out[g + min(e, need)] = j0 + r;
        ++g;
      } else if (in && k < n && (x[r] & mask) == prefix) {
        if (e < need) out[g + e] = j0 + r;
        ++e;
      }
    }
    gt_seen += tot & 0xffff;
    eq_seen += tot >> 16;
  }
}

// ===========================================================================
// Decode (stream-K): the visible pages of every (sequence, KV head) segment
// of the batch form one list, cut into equal contiguous shares, one per
// workgroup.  A share may cover the end of one segment and the start of the
// next; each covered piece yields either the final output (a segment held by
// one piece) or a normalised fp32 partial merged later by combine_kernel.
//
// Per piece, the (up to 16) query heads of the KV group are the columns of
// v_mfma_f32_16x16x32_bf16 (lane l holds operand row l % 16 and k-elements
// 8*(l/16) .. +7; result lane l holds column l % 16 and rows 4*(l/16) ..
// +3).  K rows and V^T channel rows go from HBM straight into operand
// registers.  Each 64-key chunk is four 16-key S^T blocks; block kb = 2s +
// hb, row 4u + j holds key 32 s + 8 u + 4 hb + j, so lane group u feeds keys
// 32 s + 8 u .. +7 to PV step s.
//
// The workgroup's pieces (at most 9 at a time) are laid end to end and their
// 64-key chunks cut into eight contiguous runs, one per wave.  A wave that
// reaches the end of a piece leaves its partial (max, sum, o) in its own LDS
// slot and goes on with the next piece, so no wave waits for another until
// the batch is done; then each piece is merged over the waves that touched it.
// ===========================================================================

template <int D, int P>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_kernel(DecodeArgs a) {
  constexpr int NKK = D / 32;  // k-steps of QK (32 channels each)
  constexpr int NDB = D / 16;  // 16-channel blocks of O^T
  constexpr int NW = kDecodeThreads / 64;
  constexpr int TPC = D / 4;   // merge threads per column
  constexpr int NSLOT = kDecodeSlots;
  constexpr int MAXP = NSLOT - NW + 1;  // pieces per batch: (piece, wave) pairs fit the slots
  static_assert(MAXP >= 1, "too few partial slots");
  __shared__ float s_m[NSLOT][kDecodeCols];
  __shared__ float s_l[NSLOT][kDecodeCols];
  __shared__ __attribute__((aligned(16))) float s_o[NSLOT][kDecodeCols][D];
  __shared__ __attribute__((aligned(16))) float s_rope[NW][2 * D];  // per-wave relocation table

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int c16 = lane & 15, u = lane >> 4;
  const int G = a.group;
  const int wg_end = a.wg_piece_off[blockIdx.x + 1];
  auto piece_chunks = [&](int pc) {
    const DecodeItem it = a.items[pc];
    return ((it.page_end - it.page_begin) * P + 63) / 64;
  };

  for (int b0 = a.wg_piece_off[blockIdx.x]; b0 < wg_end; b0 += MAXP) {
    const int b1 = min(wg_end, b0 + MAXP);
    int total = 0;
    for (int pc = b0; pc < b1; ++pc) total += piece_chunks(pc);
    // This wave's contiguous run of the batch's 64-key chunks, across pieces.
    const int c_end = total * (wave + 1) / NW;
    int c = total * wave / NW;
    int pc = b0, cum = 0;  // cum: first batch chunk of piece pc
    while (c < c_end) {
      int nch = piece_chunks(pc);
      while (cum + nch <= c) {
        cum += nch;
        nch = piece_chunks(++pc);
      }
      const int k0 = c - cum;                      // first chunk of the run inside piece pc
      const int k1 = min(c_end - cum, nch);        // end chunk inside piece pc
      const DecodeItem it = a.items[pc];
      const SeqDesc sd = a.seqs[it.seq];
      const SegDesc sg = a.segs[it.seq * a.num_kv_heads + it.kv_head];
      const int p = sd.kv_len - 1;
      const int W = sg.window;
      const int key_begin = sg.first_token + it.page_begin * P;
      const int key_end = sg.first_token + it.page_end * P;  // exclusive
      const int lo = max(key_begin, W > 0 ? p - W + 1 : 0);
      const int hi = min(key_end - 1, p);

      bf16x8 qv[NKK];
      {
        // Unconditional loads (lanes past the group read its last head and
        // are zeroed), so they are in flight together.
        const uint16_t *qrow =
            a.q + (static_cast<size_t>(sd.q_start) * a.num_q_heads + it.kv_head * G + min(c16, G - 1)) * D;
        if (sg.rope_off < 0) {
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 x = ld16(qrow + kk * 32 + u * 8);
            qv[kk] = as_bf16x8(c16 < G ? x : z);
          }
        } else {
          relocate_row<D, NKK>(qv, qrow, 32, u * 8, c16 < G, a.rope.tables + sg.rope_off, s_rope[wave], a.rope);
        }
      }

      f32x4 oacc[NDB];
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};
      float m = kNegInf, l = 0.f;

      // Chunks k0 .. k1-1 of the piece, each handled as two 32-key halves:
      // all loads of a chunk are issued before its two halves are computed,
      // so each wave keeps 32 KiB in flight.
      const int n_halves = 2 * (k1 - k0);
      auto half_base = [&](int j) { return key_begin + (k0 + (j >> 1)) * 64 + 32 * (j & 1); };
      auto load_half = [&](int j, u32x4 (&kb_)[2][NKK], u32x4 (&vb_)[NDB], int upage) {
        const int kbase = half_base(j);
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          const int key = kbase + 8 * (c16 >> 2) + 4 * hb + (c16 & 3);
          const int rel = key - sg.first_token;
          const bool ok = key < key_end;
          const int page = P == 64 ? upage : (ok ? a.page_ids[sg.page_off + rel / P] : 0);
          const uint16_t *krow = a.k_pool + (static_cast<size_t>(page) * P + rel % P) * D;
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (ok) x = ld16(krow + kk * 32 + u * 8);
            kb_[hb][kk] = x;
          }
        }
        const int key = kbase + 8 * u;
        const int rel = key - sg.first_token;
        const bool ok = key < key_end;
        const int page = P == 64 ? upage : (ok ? a.page_ids[sg.page_off + rel / P] : 0);
        const uint16_t *vbase = a.v_pool + static_cast<size_t>(page) * P * D + rel % P;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          u32x4 x = {0u, 0u, 0u, 0u};
          if (ok) x = ld16(vbase + static_cast<size_t>(db * 16 + c16) * P);
          vb_[db] = x;
        }
      };
      auto compute_half = [&](int j, const u32x4 (&kb_)[2][NKK], const u32x4 (&vb_)[NDB]) {
        const int kbase = half_base(j);
        f32x4 sc[2];
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
          f32x4 acc = f32x4{};
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(kb_[hb][kk]), qv[kk], acc, 0, 0, 0);
          sc[hb] = acc;
        }
        float mx = kNegInf;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int key = kbase + 8 * u + 4 * hb + jj;
            if (key < lo || key > hi) sc[hb][jj] = kNegInf;
            mx = fmaxf(mx, sc[hb][jj]);
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool bump = mx * a.scale_log2 > m * a.scale_log2 + kRescaleLog2;
        const float m_new = bump ? mx : m;
        const float msc = m_new == kNegInf ? 0.f : m_new * a.scale_log2;
        if (__any(bump)) {
          const float alpha = bump ? fast_exp2(m * a.scale_log2 - msc) : 1.f;
          l *= alpha;
#pragma unroll
          for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
        }
        m = m_new;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            sc[hb][jj] = fast_exp2(fmaf(sc[hb][jj], a.scale_log2, -msc));
            l += sc[hb][jj];
          }
        }
        const bf16x8 pb = pack8_bf16(sc[0][0], sc[0][1], sc[0][2], sc[0][3], sc[1][0], sc[1][1], sc[1][2], sc[1][3]);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
          oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(vb_[db]), pb, oacc[db], 0, 0, 0);
      };
      u32x4 kb0[2][NKK], vb0[NDB], kb1[2][NKK], vb1[NDB];
      // P == 64: a chunk is exactly one page; its id is a uniform (scalar)
      // load, fetched one chunk ahead, so no vector load of the page table
      // sits in front of the chunk's K/V loads.
      auto chunk_page = [&](int j) {
        const int pi = min((half_base(j) - sg.first_token) / P, sg.n_pages - 1);
        return a.page_ids[sg.page_off + pi];
      };
      int upage = (P == 64 && n_halves > 0) ? chunk_page(0) : 0;
      for (int j = 0; j < n_halves; j += 2) {
        const int next = (P == 64 && j + 2 < n_halves) ? chunk_page(j + 2) : 0;
        load_half(j, kb0, vb0, upage);
        load_half(j + 1, kb1, vb1, upage);
        compute_half(j, kb0, vb0);
        compute_half(j + 1, kb1, vb1);
        upage = next;
      }

      // This wave's partial of piece pc goes to its own slot: slot
      // (pc - b0) + wave is distinct for every (piece, wave) pair of a batch
      // because each wave's pieces follow the previous wave's.
      float lt = l + __shfl_xor(l, 16);
      lt += __shfl_xor(lt, 32);
      const int slot = pc - b0 + wave;
      if (u == 0) {
        s_m[slot][c16] = m;
        s_l[slot][c16] = lt;
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        *reinterpret_cast<f32x4 *>(&s_o[slot][c16][db * 16 + u * 4]) = oacc[db];
      c = cum + k1;
    }
    __syncthreads();

    // Merge each piece of the batch over the waves whose runs touched it.
    // Thread -> (column, 4 channels).  A segment held by one piece writes
    // the output; otherwise the piece writes its normalised partial.
    int pstart = 0;
    for (int pc2 = b0; pc2 < b1; ++pc2) {
      const int pend = pstart + piece_chunks(pc2);
      const DecodeItem it = a.items[pc2];
      const SeqDesc sd = a.seqs[it.seq];
      const bool single = it.n_parts == 1;
      const size_t out_row0 = static_cast<size_t>(sd.q_start) * a.num_q_heads + it.kv_head * G;
      for (int e = tid; e < G * TPC; e += kDecodeThreads) {
        const int cc = e / TPC, d0 = (e - cc * TPC) * 4;
        float mm = kNegInf;
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const bool touched = max(pstart, total * w / NW) < min(pend, total * (w + 1) / NW);
          if (touched) mm = fmaxf(mm, s_m[pc2 - b0 + w][cc]);
        }
        const float m_use = mm == kNegInf ? 0.f : mm;
        float lw = 0.f;
        f32x4 acc = f32x4{};
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const bool touched = max(pstart, total * w / NW) < min(pend, total * (w + 1) / NW);
          if (!touched) continue;
          const int sl = pc2 - b0 + w;
          const float f = fast_exp2((s_m[sl][cc] - m_use) * a.scale_log2);
          lw = fmaf(s_l[sl][cc], f, lw);
          acc += *reinterpret_cast<const f32x4 *>(&s_o[sl][cc][d0]) * f;
        }
        const float inv = lw > 0.f ? 1.f / lw : 0.f;
        const float lse_v = lw > 0.f ? mm * a.scale + logf(lw) : kNegInf;
        if (single) {
          *reinterpret_cast<u32x2 *>(a.o + (out_row0 + cc) * D + d0) =
              pack4_bf16(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
          if (d0 == 0 && a.lse) a.lse[out_row0 + cc] = lse_v;
        } else {
          *reinterpret_cast<f32x4 *>(a.part_o + (static_cast<size_t>(it.part) * kDecodeCols + cc) * D + d0) =
              acc * inv;
          if (d0 == 0) a.part_lse[static_cast<size_t>(it.part) * kDecodeCols + cc] = lse_v;
        }
      }
      pstart = pend;
    }
    __syncthreads();  // the slots are free for the next batch
  }
}

// ===========================================================================
// Combine: o = sum_s exp(lse_s - lse) o_s with lse = ln sum_s exp(lse_s);
// parts with lse_s = -inf carry weight 0.
// ===========================================================================

template <int D>
__global__ __launch_bounds__(256) void combine_kernel(CombineArgs a) {
  constexpr int TPE = D / 4;        // threads per entry
  constexpr int EPP = 256 / TPE;    // entries per pass
  constexpr int B = 4;              // parts loaded per batch
  const CombineItem it = a.items[blockIdx.x];
  const int entries = it.rows * it.heads;
  const int d0 = (threadIdx.x % TPE) * 4;
  // grid.y: groups of EPP entries, so that a long item spreads over workgroups
  for (int e = blockIdx.y * EPP + threadIdx.x / TPE; e < entries; e += EPP * gridDim.y) {
    float mm = kNegInf, wsum = 0.f;
    f32x4 acc = f32x4{};
    for (int s0 = 0; s0 < it.n_parts; s0 += B) {
      float ls[B];
      f32x4 os[B];
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const int s = min(s0 + k, it.n_parts - 1);
        const size_t slot = static_cast<size_t>(it.part_begin + s) * a.slot_rows + e;
        ls[k] = s0 + k < it.n_parts ? a.part_lse[slot] : kNegInf;
        os[k] = *reinterpret_cast<const f32x4 *>(a.part_o + slot * D + d0);
      }
      float bm = mm;
#pragma unroll
      for (int k = 0; k < B; ++k) bm = fmaxf(bm, ls[k]);
      if (bm == kNegInf) continue;
      const float r = __expf(mm - bm);  // mm = -inf gives 0
      wsum *= r;
      acc *= r;
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const float w = __expf(ls[k] - bm);
        wsum += w;
        acc += os[k] * w;
      }
      mm = bm;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int row = it.out_row + e / it.heads;
    const int h = it.head0 + e % it.heads;
    uint16_t *orow = a.o + (static_cast<size_t>(row) * a.num_q_heads + h) * D;
    *reinterpret_cast<u32x2 *>(orow + d0) = pack4_bf16(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    if (d0 == 0 && a.lse) a.lse[static_cast<size_t>(row) * a.num_q_heads + h] = wsum > 0.f ? mm + logf(wsum) : kNegInf;
  }
}

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

#define SEGKV_DISPATCH_DP(KERNEL, D, P, GRID, BLOCK, STREAM, ARGS)                                \
  do {                                                                                           \
    if ((D) == 64 && (P) == 16) hipLaunchKernelGGL((KERNEL<64, 16>), GRID, BLOCK, 0, STREAM, ARGS); \
    else if ((D) == 64 && (P) == 32) hipLaunchKernelGGL((KERNEL<64, 32>), GRID, BLOCK, 0, STREAM, ARGS); \
    else if ((D) == 64 && (P) == 64) hipLaunchKernelGGL((KERNEL<64, 64>), GRID, BLOCK, 0, STREAM, ARGS); \
    else if ((D) == 128 && (P) == 16) hipLaunchKernelGGL((KERNEL<128, 16>), GRID, BLOCK, 0, STREAM, ARGS); \
    else if ((D) == 128 && (P) == 32) hipLaunchKernelGGL((KERNEL<128, 32>), GRID, BLOCK, 0, STREAM, ARGS); \
    else if ((D) == 128 && (P) == 64) hipLaunchKernelGGL((KERNEL<128, 64>), GRID, BLOCK, 0, STREAM, ARGS); \
    else return hipErrorInvalidValue;                                                            \
  } while (0)

hipError_t launch_scatter(const ScatterArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(scatter_kernel, head_dim, page_size, dim3(n_items + a.copy_wgs), dim3(kScatterThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(prefill_kernel, head_dim, page_size, dim3(n_items), dim3(kPrefillThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_wide(const PrefillArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(prefill_wide_kernel, head_dim, page_size, dim3(n_items), dim3(kPrefillWideThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s) {
  if (n_wgs <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(decode_kernel, head_dim, page_size, dim3(n_wgs), dim3(kDecodeThreads), s, a);
  return hipGetLastError();
}

// Copy of the per-call tables from pinned host memory to device memory.
__global__ __launch_bounds__(256) void upload_kernel(uint4 *dst, const uint4 *src, size_t n16) {
  const size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x;
  if (i < n16) dst[i] = src[i];
}

// Device scratch of segkv_decode_noalloc: its tables and split partials,
// one array per GPU for the life of the process.  Host code never uses the
// array's name as a device address; scratch_address() resolves the device
// copy of the current GPU once and hands out that pointer.
constexpr int kMaxScratchDevices = 64;
static __device__ __attribute__((aligned(256))) unsigned char scratch[kStaticScratchBytes];

hipError_t scratch_address(void **out) {
  static std::mutex mu;
  static void *ptr[kMaxScratchDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    ptr[dev] = p;
  }
  *out = ptr[dev];
  return hipSuccess;
}

hipError_t launch_upload(void *dst, const void *src_pinned, size_t bytes, hipStream_t s) {
  const size_t n16 = (bytes + 15) / 16;
  if (n16 == 0) return hipSuccess;
  hipLaunchKernelGGL(upload_kernel, dim3(static_cast<unsigned>((n16 + 255) / 256)), dim3(256), 0, s,
                     static_cast<uint4 *>(dst), static_cast<const uint4 *>(src_pinned), n16);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, int n_items, int max_entries, int head_dim, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  const int epp = 256 / (head_dim / 4);
  const dim3 grid(n_items, (max_entries + epp - 1) / epp);
  if (head_dim == 64) hipLaunchKernelGGL(combine_kernel<64>, grid, dim3(256), 0, s, a);
  else if (head_dim == 128) hipLaunchKernelGGL(combine_kernel<128>, grid, dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_score(const ScoreArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(score_kernel, head_dim, page_size, dim3(n_items), dim3(kPrefillThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_score_reduce(const ScoreReduceArgs &a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(score_reduce_kernel, dim3(a.n_rows), dim3(64 * kReduceWaves), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, int n_seqs, hipStream_t s) {
  if (n_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(topk_kernel, dim3(n_seqs), dim3(kTopkThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_merge(const MergeArgs &a, int n_wgs, int head_dim, hipStream_t s) {
  if (n_wgs <= 0 || a.n_pairs <= 0) return hipSuccess;
  if (head_dim == 64) hipLaunchKernelGGL(merge_kernel<64>, dim3(n_wgs), dim3(kMergeThreads), 0, s, a);
  else if (head_dim == 128) hipLaunchKernelGGL(merge_kernel<128>, dim3(n_wgs), dim3(kMergeThreads), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace segkv
