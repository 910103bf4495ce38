// HIP kernels of libsegkv: attention-mass token scores and their top-k.

#include "kernels_common.h"
#include "page_layout.h"
#include "segkv_launch.h"

namespace segkv {
namespace {

// ===========================================================================
// Attention-mass token scores ("attention as a router" for the sparse FFN:
// "Xiaohongshu Open-Sources RedKnot" page, "What Happened" item 2; "RedKnot:
// Head-Aware KV Reuse and SegPagedAttention" page, "The Three Core
// Mechanisms in Detail", second mechanism).  A second pass over the prefill's
// work: with the rows' final LSE known, key j receives sum over rows (t, h)
// of exp(scale q.k_j - lse).  The product is taken as S = Q K^T (operands of
// the prefill's S^T swapped), so a lane holds one key column and 16 query
// rows per 32-row block and the sum over queries is in-lane plus one
// lane-pair swap.  A workgroup covers the prefill's 256 rows with 4 waves
// of 64 rows (two blocks, so each K operand read from LDS feeds two
// products), and two workgroups share a CU.  The waves' per-tile key sums
// meet in a double-buffered LDS exchange that rides on the K pipeline's
// per-tile barrier; one wave writes the tile's 64 sums as a partial row.
// Partial rows are added by score_reduce_kernel in a fixed order, so the
// scores do not depend on the work order.  The grid is persistent (one
// workgroup per resident slot) and takes the pieces from a queue.
// ===========================================================================

constexpr int kScoreThreads = 256;  // 4 waves of 64 rows: two workgroups per CU

template <int D, int P>
__global__ __launch_bounds__(kScoreThreads, 2) void score_kernel(ScoreArgs a) {
  using L = PrefillLds<D>;
  using PL = PageLayout<D, P>;
  constexpr int NKK = D / 16;
  constexpr int NW = kScoreThreads / 64;
  constexpr int RB = 2;  // 32-row blocks per wave: each K operand read feeds RB products
  constexpr int K_INSTR = L::K_CHUNKS / kScoreThreads;
  constexpr int NSTAGE = 4;  // K tiles in LDS: the one read and NSTAGE - 1 in flight
  constexpr int AHEAD = NSTAGE - 1;
  constexpr int KSTAGE = L::K_CHUNKS * 16;  // bytes of one K tile
  constexpr float kLog2e = 1.4426950408889634f;
  static_assert(kPrefillRows == 32 * RB * NW && K_INSTR >= 1 && L::K_CHUNKS % kScoreThreads == 0, "tile layout");
  __shared__ __attribute__((aligned(16))) uint4 smem4[NSTAGE * KSTAGE / 16];
  __shared__ float sx[2][NW][kTileKeys];
  __shared__ __attribute__((aligned(16))) float s_rope[NW][2 * D];  // per-wave relocation table
  char *smem = reinterpret_cast<char *>(smem4);

  const int G = a.group;
  const int rows = a.rows_per_tile;
  // Work queue: workgroup w starts with item w, and each item fetches the
  // index of this workgroup's next one (thread 0's atomic, issued at the
  // item's start and handed over through LDS at its end, alternating two
  // slots so that a slot is rewritten only after a later barrier).  Between
  // two items the barrier ending an item and the one after the next item's
  // first loads keep the K stages and the sum exchange apart.
  __shared__ int s_next[2];
  int ii = blockIdx.x;
  for (int slot = 0; ii < a.n_items; slot ^= 1) {
    // The thread index passes an empty asm statement per item, so values
    // derived from it are rebuilt per item rather than held in registers
    // across items.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, wave = tid >> 6;
    const int col = lane & 31, half = lane >> 5;
    const PrefillItem it = sload(a.items + ii);
    int nxt = 0;
    if (tid == 0) nxt = atomicAdd(a.counter, 1);
    const SeqDesc sd = sload(a.seqs + it.seq);
    const SegDesc sg = sload(a.segs + it.seq * a.num_kv_heads + it.kv_head);
    const int t0 = it.qtile * rows;
    const int t_last = min(t0 + rows, sd.q_len) - 1;
    const int base = sd.kv_len - sd.q_len;
    const int W = sg.window;
    const int p_wmin = base + min(t0 + (wave * 64) / G, t_last);
    const int p_wmax = base + min(t0 + (wave * 64 + 63) / G, t_last);

    // Q operands (A of S = Q K^T): in block b this lane supplies query row
    // 64 wave + 32 b + col.  Loads are unconditional (an invalid row reads the
    // tile's last valid row and is zeroed afterwards), so they are in flight
    // together.
    bf16x8 qv[RB][NKK];
    float lse_own[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) {
      const int r = wave * 64 + 32 * b + col;
      const int po = r / G;
      const int h = it.kv_head * G + (r - po * G);
      const int t = t0 + po;
      const bool valid = po < rows && t < sd.q_len;
      const size_t qi = static_cast<size_t>(sd.q_start + min(t, t_last)) * a.num_q_heads + h;
      if (sg.rope_off < 0) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) {
          const u32x4 z = {0u, 0u, 0u, 0u};
          const u32x4 x = ld16(a.q + qi * D + kk * 16 + half * 8);
          qv[b][kk] = as_bf16x8(valid ? x : z);
        }
      } else {
        relocate_row<D, NKK>(qv[b], a.q + qi * D, 16, half * 8, valid, a.rope.tables + sg.rope_off, s_rope[wave],
                             a.rope);
      }
      // Rows past the chunk get lse = +inf, hence probability 0.
      lse_own[b] = valid ? a.lse[qi] * kLog2e : __builtin_inff();
    }
    // The rows of S this lane holds: in block b, register v is row
    // n = 64 wave + 32 b + 8 (v/4) + 4 half + v%4 of the workgroup; its LSE
    // comes from the lane that loaded it.  Its query position minus t0,
    // min(n / G, t_last - t0) (below rows <= 256), is kept as byte v%4 of
    // pos4[b][v/4].  n / G is taken in fp32: with n < 256 and G <= 256,
    // (n + 1/2) / G lies at least 1/(2G) from an integer, far above the
    // rounding error, so truncation gives the integer quotient.
    float lse2[RB][16];
    uint32_t pos4[RB][4];
    {
      const float rg = 1.f / static_cast<float>(G);
      const int rel_max = t_last - t0;
#pragma unroll
      for (int b = 0; b < RB; ++b) {
        const float nb = static_cast<float>(wave * 64 + 32 * b + 4 * half) + 0.5f;
#pragma unroll
        for (int q = 0; q < 4; ++q) pos4[b][q] = 0u;
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rw = 8 * (v >> 2) + 4 * half + (v & 3);
          lse2[b][v] = __shfl(lse_own[b], rw);
          const int quo = static_cast<int>((nb + static_cast<float>(8 * (v >> 2) + (v & 3))) * rg);
          pos4[b][v >> 2] |= static_cast<uint32_t>(min(quo, rel_max)) << (8 * (v & 3));
        }
      }
    }
    // Wait for Q and the LSE values once, here; inside the tile loop the
    // compiler would otherwise wait for every outstanding load (the
    // prefetched tiles included) before their first use in each tile.
#pragma unroll
    for (int b = 0; b < RB; ++b) {
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qv[b][kk]));
#pragma unroll
      for (int v = 0; v < 16; ++v) asm volatile("" : "+v"(lse2[b][v]));
    }

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
          lds_dma16_s(a.k_pool + static_cast<size_t>(pid[0]) * (P * D), static_cast<uint32_t>(PL::k_elem(row, logical) * 2),
                      st + (j * NW + wave) * 1024);
        } else {
          const int rel = k0 + row - sg.first_token;
          const int slot = rel >= 0 && rel / P <= last_page ? row % P : 0;
          int page = pid[0];
#pragma unroll
          for (int i = 1; i < NP; ++i)
            if (row / P == i) page = pid[i];
          lds_dma16(a.k_pool + static_cast<size_t>(page) * (P * D) + PL::k_elem(slot, logical), st + (j * NW + wave) * 1024);
        }
      }
    };

    const int kswz = L::k_swz(col);  // keys col and col + 32 share it
    // Entry (row, key) is visible iff prow - W < key <= prow (W = 0: key <=
    // prow): with d = prow - key taken as unsigned, iff d < wlim.
    const uint32_t wlim = W > 0 ? static_cast<uint32_t>(W) : 0x80000000u;
    // Masked scores become -inf, hence probability 0 whatever the row's LSE.
    auto apply_mask = [&](f32x16 (&s)[RB], int key) {
      const int krel = key - base - t0;  // prow - key = (position - t0) - krel
      // (opaque here, so that the compiler keeps no per-entry differences
      // live across the tile loop)
#pragma unroll
      for (int b = 0; b < RB; ++b) {
#pragma unroll
        for (int q = 0; q < 4; ++q) asm volatile("" : "+v"(pos4[b][q]));
      }
#pragma unroll
      for (int b = 0; b < RB; ++b) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int rel = static_cast<int>(__builtin_amdgcn_ubfe(pos4[b][v >> 2], 8 * (v & 3), 8));
          if (static_cast<uint32_t>(rel - krel) >= wlim) s[b][v] = kNegInf;
        }
      }
    };
    // Each wave keeps its matrix cores and its vector ALU busy together: a
    // half step runs the RB x NKK products of one 32-key half of a tile (keys
    // k0 + 32 hk + col, from the stage at st) into acc, each K operand read
    // feeding RB of them, and between them the exponentials and the row sum
    // of the scores prev of the half before it, which no product of this step
    // reads.  Returns that half's key sums over this wave's 64 rows (both
    // lanes of a pair end with the full sum).
    constexpr int VPK = RB * 16 / NKK;  // entries of prev per K operand
    constexpr int KAHEAD = 2;           // K operand reads in flight ahead of the products
    auto half_step = [&](const char *st, int hk, f32x16 (&acc)[RB], const f32x16 (&prev)[RB]) -> float {
      const char *kb = st + (col + 32 * hk) * L::KCPR * 16;
      bf16x8 kr[NKK];
      auto kread = [&](int kk) {
        kr[kk] = as_bf16x8(*reinterpret_cast<const u32x4 *>(kb + ((2 * kk + half) ^ kswz) * 16));
      };
#pragma unroll
      for (int kk = 0; kk < KAHEAD; ++kk) kread(kk);
      f32x16 s[RB];
#pragma unroll
      for (int b = 0; b < RB; ++b) s[b] = f32x16{};
      float e = 0.f;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        // Empty asm statements pin the program order (the products of k-step
        // kk, the next operand read, then entries of prev under the
        // products); pure arithmetic would otherwise drift to its first use.
        asm volatile("" : "+v"(kr[kk]));
#pragma unroll
        for (int b = 0; b < RB; ++b) s[b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qv[b][kk], kr[kk], s[b], 0, 0, 0);
        if (kk + KAHEAD < NKK) kread(kk + KAHEAD);
#pragma unroll
        for (int j = 0; j < VPK; ++j) {
          const int m = kk * VPK + j;  // entries in the order (block, register)
          e += fast_exp2(fmaf(prev[m / 16][m % 16], a.scale_log2, -lse2[m / 16][m % 16]));
        }
        asm volatile("" : "+v"(e));
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int b = 0; b < RB; ++b) acc[b] = s[b];
      return e + __shfl_xor(e, 32);
    };
    // Tile i's sums of all waves are in sx[i % 2] after the barrier ending
    // iteration i + 1; wave i % NW adds them (fixed order) during iteration
    // i + 2 (or after the loop).
    auto flush = [&](int i) {
      if (wave == i % NW) {
        float acc = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) acc += sx[i & 1][w][lane];
        a.part[(static_cast<size_t>(it.part) + i) * kTileKeys + lane] = acc;
      }
    };
    // Whether every entry of this wave's rows against tile k0 is visible.
    // Masked entries are still multiplied (they give 0).
    auto tile_full = [&](int k0) {
      return k0 + kTileKeys - 1 <= p_wmin && (W == 0 || k0 >= p_wmax - W + 1);
    };

    constexpr int LOADS_PER_TILE = K_INSTR;
    static_assert(AHEAD >= 1 && AHEAD <= 4, "wait counts below");
    // Waits until at most `pending` tiles' loads are in flight (loads land in
    // issue order), then meets the other waves: barriers leave the newest
    // tiles' loads in flight (see the prefill).
    auto wait_barrier = [&](int pending) {
      if (pending >= 3)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(3 * LOADS_PER_TILE) : "memory");
      else if (pending == 2)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOADS_PER_TILE) : "memory");
      else if (pending == 1)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    const int tb = it.tile_begin, te = it.tile_end;
    if (tb >= te) {  // (the host cuts no empty pieces; the hand-over stays uniform)
      if (tid == 0) s_next[slot] = nxt + static_cast<int>(gridDim.x);
      __syncthreads();
      ii = __builtin_amdgcn_readfirstlane(s_next[slot]);
      continue;
    }
    for (int j = 0; j < AHEAD && tb + j < te; ++j) issue_tile(tb + j, j);
    wait_barrier(min(AHEAD, te - tb) - 1);
    // sa / sb: scores of the current tile's first / second key half.  The
    // second half of tile i is exponentiated during the first half step of
    // tile i + 1 (at the first tile, during a step over zeros whose sum is
    // dropped), so tile i's sums go to sx one iteration late.
    f32x16 sa[RB], sb[RB];
#pragma unroll
    for (int b = 0; b < RB; ++b) sa[b] = sb[b] = f32x16{};
    float c0 = 0.f;
    bool full_prev = true;
    for (int tile = tb; tile < te; ++tile) {
      const int i = tile - tb;
      if (tile + AHEAD < te) issue_tile(tile + AHEAD, (i + AHEAD) % NSTAGE);
      if (i >= 2) flush(i - 2);
      const char *st = smem + (i % NSTAGE) * KSTAGE;
      const int k0 = tile * kTileKeys;
      const bool full = tile_full(k0);
      if (!full_prev) apply_mask(sb, k0 - 32 + col);
      const float c1 = half_step(st, 0, sa, sb);
      if (i >= 1) sx[(i - 1) & 1][wave][half * 32 + col] = half ? c1 : c0;
      if (!full) apply_mask(sa, k0 + col);
      c0 = half_step(st, 1, sb, sa);
      full_prev = full;
      wait_barrier(min(AHEAD, te - 1 - tile) - 1);  // tile + 1 has landed
    }
    const int n = te - tb;
    if (n >= 2) flush(n - 2);
    if (!full_prev) apply_mask(sb, te * kTileKeys - 32 + col);
    float e = 0.f;
#pragma unroll
    for (int m = 0; m < RB * 16; ++m) e += fast_exp2(fmaf(sb[m / 16][m % 16], a.scale_log2, -lse2[m / 16][m % 16]));
    const float c1 = e + __shfl_xor(e, 32);
    sx[(n - 1) & 1][wave][half * 32 + col] = half ? c1 : c0;
    if (tid == 0) s_next[slot] = nxt + static_cast<int>(gridDim.x);
    __syncthreads();
    flush(n - 1);
    ii = __builtin_amdgcn_readfirstlane(s_next[slot]);
  }
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

}  // namespace

hipError_t launch_score(const ScoreArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s) {
  if (n_wgs <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(score_kernel, head_dim, page_size, dim3(n_wgs), dim3(kScoreThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_score_reduce(const ScoreReduceArgs &a, hipStream_t s) {
  if (a.n_rows <= 0) return hipSuccess;
  SEGKV_LAUNCH(score_reduce_kernel, dim3(a.n_rows), dim3(64 * kReduceWaves), s, a);
  return hipGetLastError();
}

hipError_t launch_topk(const TopkArgs &a, int n_seqs, hipStream_t s) {
  if (n_seqs <= 0) return hipSuccess;
  SEGKV_LAUNCH(topk_kernel, dim3(n_seqs), dim3(kTopkThreads), s, a);
  return hipGetLastError();
}

}  // namespace segkv
