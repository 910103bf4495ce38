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

#include "segkv_internal.h"

namespace segkv {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kNegInf = -__builtin_inff();

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

// ===========================================================================
// Scatter: copy newly appended K/V rows into their pages.
// ===========================================================================

template <int D, int P>
__global__ __launch_bounds__(kScatterThreads) void scatter_kernel(ScatterArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t sv[P * D];
  const ScatterItem it = a.items[blockIdx.x];
  const int tid = threadIdx.x;
  constexpr int CPR = D / 8;  // 16-byte chunks per row
  const int n_rows = it.slot_end - it.slot_begin;
  uint16_t *kpage = a.k_pool + static_cast<size_t>(it.page_id) * P * D;
  uint16_t *vpage = a.v_pool + static_cast<size_t>(it.page_id) * P * D;

  // K rows, and V rows staged in LDS for the transpose.
  for (int c = tid; c < n_rows * CPR; c += kScatterThreads) {
    const int row = c / CPR, dc = c - row * CPR;
    const size_t src = (static_cast<size_t>(it.src_row + row) * a.num_kv_heads + it.kv_head) * D + dc * 8;
    *reinterpret_cast<u32x4 *>(kpage + static_cast<size_t>(it.slot_begin + row) * D + dc * 8) = ld16(a.k_new + src);
    *reinterpret_cast<u32x4 *>(sv + (it.slot_begin + row) * D + dc * 8) = ld16(a.v_new + src);
  }
  if (it.zero_tail) {
    const u32x4 z = {0u, 0u, 0u, 0u};
    for (int c = tid; c < (P - it.slot_end) * CPR; c += kScatterThreads) {
      const int row = c / CPR, dc = c - row * CPR;
      *reinterpret_cast<u32x4 *>(kpage + static_cast<size_t>(it.slot_end + row) * D + dc * 8) = z;
      *reinterpret_cast<u32x4 *>(sv + (it.slot_end + row) * D + dc * 8) = z;
    }
  }
  __syncthreads();
  // V^T rows: channel d holds slots [slot_begin, wend) contiguously.
  const int wend = it.zero_tail ? P : it.slot_end;
  const int n = wend - it.slot_begin;
  if ((it.slot_begin & 7) == 0 && (n & 7) == 0) {
    const int cpr = n / 8;
    for (int c = tid; c < D * cpr; c += kScatterThreads) {
      const int d = c / cpr, s0 = it.slot_begin + (c - d * cpr) * 8;
      uint16_t tmp[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) tmp[e] = sv[(s0 + e) * D + d];
      *reinterpret_cast<u32x4 *>(vpage + static_cast<size_t>(d) * P + s0) = *reinterpret_cast<const u32x4 *>(tmp);
    }
  } else {
    for (int c = tid; c < D * n; c += kScatterThreads) {
      const int d = c / n, s = it.slot_begin + (c - d * n);
      vpage[static_cast<size_t>(d) * P + s] = sv[s * D + d];
    }
  }
}

// ===========================================================================
// Prefill: one workgroup = 128 (query position, query head) rows of one
// (sequence, KV head) over a range of 64-key tiles.
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

template <int D, int P>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillArgs a) {
  constexpr int KS = D + 8;          // LDS row stride of the K tile (elements)
  constexpr int VS = kTileKeys + 8;  // LDS row stride of the V^T tile
  constexpr int NKK = D / 16;        // k-steps of the QK product
  constexpr int NDB = D / 32;        // 32-channel blocks of O^T
  constexpr int KCH = kTileKeys * D / 8;
  constexpr int KPT = KCH / kPrefillThreads;  // 16-byte K chunks per thread per tile
  constexpr int VPT = KCH / kPrefillThreads;  // same count for V^T
  __shared__ __attribute__((aligned(16))) uint16_t sK[kTileKeys * KS];
  __shared__ __attribute__((aligned(16))) uint16_t sV[D * VS];

  const PrefillItem it = a.items[blockIdx.x];
  const SeqDesc sd = a.seqs[it.seq];
  const SegDesc sg = a.segs[it.seq * a.num_kv_heads + it.kv_head];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 31, half = lane >> 5;
  const int G = a.group;
  const int rows = a.rows_per_tile;

  // Query row of this lane's column.
  const int r = wave * 32 + col;
  const int pos_off = r / G;
  const int h = it.kv_head * G + (r - pos_off * G);
  const int t0 = it.qtile * rows;
  const int t_last = min(t0 + rows, sd.q_len) - 1;  // last valid query of the tile
  const int t = t0 + pos_off;
  const bool valid = pos_off < rows && t < sd.q_len;
  const int base = sd.kv_len - sd.q_len;
  const int p = base + min(t, t_last);  // invalid columns mimic the last valid row
  const int W = sg.window;
  const int vis_lo = W > 0 ? p - W + 1 : 0;
  // Wave-wide position range (positions grow with r).
  const int p_wmin = base + min(t0 + (wave * 32) / G, t_last);
  const int p_wmax = base + min(t0 + (wave * 32 + 31) / G, t_last);

  // Q^T operand, held in registers for the whole item.
  bf16x8 qv[NKK];
  {
    const uint16_t *qrow = a.q + (static_cast<size_t>(sd.q_start + t) * a.num_q_heads + h) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (valid) x = ld16(qrow + kk * 16 + half * 8);
      qv[kk] = as_bf16x8(x);
    }
  }

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m = kNegInf;  // running max of raw scores of this column
  float l = 0.f;      // this lane's share of the running sum

  u32x4 kreg[KPT], vreg[VPT];
  auto load_tile = [&](int tile) {
    const int k0 = tile * kTileKeys;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int chunk = tid + i * kPrefillThreads;
      const int key = chunk / (D / 8), dc = chunk % (D / 8);
      const int rel = k0 + key - sg.first_token;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (rel >= 0 && rel / P < sg.n_pages) {
        const int page = a.page_ids[sg.page_off + rel / P];
        x = ld16(a.k_pool + (static_cast<size_t>(page) * P + rel % P) * D + dc * 8);
      }
      kreg[i] = x;
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int chunk = tid + i * kPrefillThreads;
      const int d = chunk / (kTileKeys / 8), kc = chunk % (kTileKeys / 8);
      const int rel = k0 + kc * 8 - sg.first_token;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (rel >= 0 && rel / P < sg.n_pages) {
        const int page = a.page_ids[sg.page_off + rel / P];
        x = ld16(a.v_pool + static_cast<size_t>(page) * P * D + static_cast<size_t>(d) * P + rel % P);
      }
      vreg[i] = x;
    }
  };

  const int key_a0 = st_row_key(col);  // K row this lane feeds to block 0 (block 1: +32)

  if (it.tile_begin < it.tile_end) load_tile(it.tile_begin);
  for (int tile = it.tile_begin; tile < it.tile_end; ++tile) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int chunk = tid + i * kPrefillThreads;
      *reinterpret_cast<u32x4 *>(sK + (chunk / (D / 8)) * KS + (chunk % (D / 8)) * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
      const int chunk = tid + i * kPrefillThreads;
      *reinterpret_cast<u32x4 *>(sV + (chunk / (kTileKeys / 8)) * VS + (chunk % (kTileKeys / 8)) * 8) = vreg[i];
    }
    __syncthreads();
    if (tile + 1 < it.tile_end) load_tile(tile + 1);

    const int k0 = tile * kTileKeys;
    const bool empty = k0 > p_wmax || (W > 0 && k0 + kTileKeys - 1 < p_wmin - W + 1);
    if (empty) continue;
    const bool full = k0 + kTileKeys - 1 <= p_wmin && (W == 0 || k0 >= p_wmax - W + 1);

    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      const bf16x8 ka0 = as_bf16x8(*reinterpret_cast<const u32x4 *>(sK + key_a0 * KS + kk * 16 + half * 8));
      const bf16x8 ka1 = as_bf16x8(*reinterpret_cast<const u32x4 *>(sK + (key_a0 + 32) * KS + kk * 16 + half * 8));
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka0, qv[kk], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka1, qv[kk], s1, 0, 0, 0);
    }
    if (!full) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = k0 + ((v >> 3) << 4) + (half << 3) + (v & 7);
        if (key < vis_lo || key > p) s0[v] = kNegInf;
        if (key + 32 < vis_lo || key + 32 > p) s1[v] = kNegInf;
      }
    }
    float mx = kNegInf;
#pragma unroll
    for (int v = 0; v < 16; ++v) mx = fmaxf(mx, fmaxf(s0[v], s1[v]));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f((m - m_use) * a.scale_log2);
    const float msc = m_use * a.scale_log2;
    float lsum = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      s0[v] = exp2f(fmaf(s0[v], a.scale_log2, -msc));
      s1[v] = exp2f(fmaf(s1[v], a.scale_log2, -msc));
      lsum += s0[v] + s1[v];
    }
    l = fmaf(l, alpha, lsum);
    m = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x16 &sv = kb ? s1 : s0;
        const bf16x8 pb = pack8_bf16(sv[8 * s + 0], sv[8 * s + 1], sv[8 * s + 2], sv[8 * s + 3], sv[8 * s + 4],
                                     sv[8 * s + 5], sv[8 * s + 6], sv[8 * s + 7]);
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          const bf16x8 va = as_bf16x8(
              *reinterpret_cast<const u32x4 *>(sV + (db * 32 + col) * VS + kb * 32 + s * 16 + half * 8));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, oacc[db], 0, 0, 0);
        }
      }
    }
  }

  const float l_tot = l + __shfl_xor(l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse_val = l_tot > 0.f ? m * a.scale + logf(l_tot) : kNegInf;
  if (it.part < 0) {
    if (!valid) return;
    uint16_t *orow = a.o + (static_cast<size_t>(sd.q_start + t) * a.num_q_heads + h) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + i * 8 + half * 4;
        *reinterpret_cast<u32x2 *>(orow + d0) =
            pack4_bf16(oacc[db][4 * i] * inv, oacc[db][4 * i + 1] * inv, oacc[db][4 * i + 2] * inv,
                       oacc[db][4 * i + 3] * inv);
      }
    }
    if (half == 0 && a.lse) a.lse[static_cast<size_t>(sd.q_start + t) * a.num_q_heads + h] = lse_val;
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
}

// ===========================================================================
// Decode: one workgroup streams pages [page_begin, page_end) of one segment
// for the (up to 16) query heads of its KV group.  Operands are loaded from
// HBM straight into registers in the v_mfma_f32_16x16x32_bf16 layout (lane l
// holds operand row l % 16 and k-elements 8*(l/16) .. +7; result lane l holds
// column l % 16 and rows 4*(l/16) .. +3).  Each 64-key chunk is four 16-key
// S^T blocks; block kb = 2s + hb, row 4u + j holds key 32 s + 8 u + 4 hb + j,
// so lane group u feeds keys 32 s + 8 u .. +7 to PV step s.  The four waves
// take chunks round-robin and are merged through LDS at the end.
// ===========================================================================

template <int D, int P>
__global__ __launch_bounds__(kDecodeThreads, 2) void decode_kernel(DecodeArgs a) {
  constexpr int NKK = D / 32;  // k-steps of QK (32 channels each)
  constexpr int NDB = D / 16;  // 16-channel blocks of O^T
  constexpr int NW = kDecodeThreads / 64;
  __shared__ float s_m[NW][kDecodeCols];
  __shared__ float s_l[NW][kDecodeCols];
  __shared__ __attribute__((aligned(16))) float s_o[NW][kDecodeCols][D];

  const DecodeItem it = a.items[blockIdx.x];
  const SeqDesc sd = a.seqs[it.seq];
  const SegDesc sg = a.segs[it.seq * a.num_kv_heads + it.kv_head];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int c16 = lane & 15, u = lane >> 4;
  const int G = a.group;

  const int p = sd.kv_len - 1;
  const int W = sg.window;
  const int key_begin = sg.first_token + it.page_begin * P;
  const int key_end = sg.first_token + it.page_end * P;  // exclusive
  const int lo = max(key_begin, W > 0 ? p - W + 1 : 0);
  const int hi = min(key_end - 1, p);

  bf16x8 qv[NKK];
  {
    const uint16_t *qrow = a.q + (static_cast<size_t>(sd.q_start) * a.num_q_heads + it.kv_head * G + c16) * D;
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (c16 < G) x = ld16(qrow + kk * 32 + u * 8);
      qv[kk] = as_bf16x8(x);
    }
  }

  f32x4 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x4{};
  float m = kNegInf, l = 0.f;

  const int n_chunks = (key_end - key_begin + 63) / 64;
  for (int ch = wave; ch < n_chunks; ch += NW) {
    const int k0 = key_begin + ch * 64;
    // K operand rows of the four S^T blocks.
    u32x4 ka[4][NKK];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int key = k0 + 32 * (kb >> 1) + 8 * (c16 >> 2) + 4 * (kb & 1) + (c16 & 3);
      const int rel = key - sg.first_token;
      const bool ok = key < key_end && rel / P < sg.n_pages;
      const int page = ok ? a.page_ids[sg.page_off + rel / P] : 0;
      const uint16_t *krow = a.k_pool + (static_cast<size_t>(page) * P + rel % P) * D;
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (ok) x = ld16(krow + kk * 32 + u * 8);
        ka[kb][kk] = x;
      }
    }
    // V^T operand: channel rows, 8 keys per lane group and PV step.
    u32x4 va[2][NDB];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int key = k0 + 32 * s + 8 * u;
      const int rel = key - sg.first_token;
      const bool ok = key < key_end && rel / P < sg.n_pages;
      const int page = ok ? a.page_ids[sg.page_off + rel / P] : 0;
      const uint16_t *vbase = a.v_pool + static_cast<size_t>(page) * P * D + rel % P;
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        u32x4 x = {0u, 0u, 0u, 0u};
        if (ok) x = ld16(vbase + static_cast<size_t>(db * 16 + c16) * P);
        va[s][db] = x;
      }
    }
    f32x4 sc[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      f32x4 acc = f32x4{};
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(ka[kb][kk]), qv[kk], acc, 0, 0, 0);
      sc[kb] = acc;
    }
    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = k0 + 32 * (kb >> 1) + 8 * u + 4 * (kb & 1) + j;
        if (key < lo || key > hi) sc[kb][j] = kNegInf;
        mx = fmaxf(mx, sc[kb][j]);
      }
    }
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m, mx);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = exp2f((m - m_use) * a.scale_log2);
    const float msc = m_use * a.scale_log2;
    float lsum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        sc[kb][j] = exp2f(fmaf(sc[kb][j], a.scale_log2, -msc));
        lsum += sc[kb][j];
      }
    }
    l = fmaf(l, alpha, lsum);
    m = m_new;
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const bf16x8 pb = pack8_bf16(sc[2 * s][0], sc[2 * s][1], sc[2 * s][2], sc[2 * s][3], sc[2 * s + 1][0],
                                   sc[2 * s + 1][1], sc[2 * s + 1][2], sc[2 * s + 1][3]);
#pragma unroll
      for (int db = 0; db < NDB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(va[s][db]), pb, oacc[db], 0, 0, 0);
    }
  }

  // Per-wave column statistics, then merge the waves through LDS.
  float lt = l + __shfl_xor(l, 16);
  lt += __shfl_xor(lt, 32);
  if (u == 0) {
    s_m[wave][c16] = m;
    s_l[wave][c16] = lt;
  }
#pragma unroll
  for (int db = 0; db < NDB; ++db)
    *reinterpret_cast<f32x4 *>(&s_o[wave][c16][db * 16 + u * 4]) = oacc[db];
  __syncthreads();

  // Thread -> (column, 4 channels); D/4 threads per column.
  constexpr int TPC = D / 4;
  for (int e = tid; e < G * TPC; e += kDecodeThreads) {
    const int cc = e / TPC, d0 = (e - cc * TPC) * 4;
    float mm = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) mm = fmaxf(mm, s_m[w][cc]);
    const float m_use = mm == kNegInf ? 0.f : mm;
    float lw = 0.f;
    f32x4 acc = f32x4{};
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float f = exp2f((s_m[w][cc] - m_use) * a.scale_log2);
      lw = fmaf(s_l[w][cc], f, lw);
      acc += *reinterpret_cast<const f32x4 *>(&s_o[w][cc][d0]) * f;
    }
    const float inv = lw > 0.f ? 1.f / lw : 0.f;
    *reinterpret_cast<f32x4 *>(a.part_o + (static_cast<size_t>(it.part) * kDecodeCols + cc) * D + d0) = acc * inv;
    if (d0 == 0)
      a.part_lse[static_cast<size_t>(it.part) * kDecodeCols + cc] = lw > 0.f ? mm * a.scale + logf(lw) : kNegInf;
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
  const CombineItem it = a.items[blockIdx.x];
  const int entries = it.rows * it.heads;
  const int d0 = (threadIdx.x % TPE) * 4;
  for (int e = threadIdx.x / TPE; e < entries; e += EPP) {
    float mm = kNegInf;
    for (int s = 0; s < it.n_parts; ++s)
      mm = fmaxf(mm, a.part_lse[static_cast<size_t>(it.part_begin + s) * a.slot_rows + e]);
    const float m_use = mm == kNegInf ? 0.f : mm;
    float wsum = 0.f;
    f32x4 acc = f32x4{};
    for (int s = 0; s < it.n_parts; ++s) {
      const size_t slot = static_cast<size_t>(it.part_begin + s) * a.slot_rows + e;
      const float w = __expf(a.part_lse[slot] - m_use);
      wsum += w;
      acc += *reinterpret_cast<const f32x4 *>(a.part_o + slot * D + d0) * w;
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const int row = it.out_row + e / it.heads;
    const int h = it.head0 + e % it.heads;
    uint16_t *orow = a.o + (static_cast<size_t>(row) * a.num_q_heads + h) * D;
    *reinterpret_cast<u32x2 *>(orow + d0) = pack4_bf16(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
    if (d0 == 0 && a.lse) a.lse[static_cast<size_t>(row) * a.num_q_heads + h] = wsum > 0.f ? mm + logf(wsum) : kNegInf;
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
  SEGKV_DISPATCH_DP(scatter_kernel, head_dim, page_size, dim3(n_items), dim3(kScatterThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(prefill_kernel, head_dim, page_size, dim3(n_items), dim3(kPrefillThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(decode_kernel, head_dim, page_size, dim3(n_items), dim3(kDecodeThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, int n_items, int head_dim, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  if (head_dim == 64) hipLaunchKernelGGL(combine_kernel<64>, dim3(n_items), dim3(256), 0, s, a);
  else if (head_dim == 128) hipLaunchKernelGGL(combine_kernel<128>, dim3(n_items), dim3(256), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace segkv
