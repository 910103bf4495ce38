// HIP kernels of libsegkv: split-KV decode, the log-sum-exp combine, and the
// fixed device scratch of the decode entry point that allocates nothing.

#include "kernels_common.h"
#include "page_layout.h"
#include "segkv_launch.h"

#include <mutex>

namespace segkv {
namespace {

// ===========================================================================
// Decode (stream-K): the visible pages of every (sequence, KV head) segment
// of the batch form one list, cut into equal contiguous shares, one per
// workgroup.  A share may cover the end of one segment and the start of the
// next; each covered piece yields either the final output (a segment held by
// one piece) or a normalised fp32 partial merged later by combine_kernel.
//
// Per piece, the query heads of one block of the KV group (up to 16; a
// larger group is split into blocks by the host) are the columns of
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
  using PL = PageLayout<D, P>;
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
      const int nh = min(kDecodeCols, G - it.head0);  // query heads (columns) of this item
      const int p = sd.kv_len - 1;
      const int W = sg.window;
      const int key_begin = sg.first_token + it.page_begin * P;
      const int key_end = sg.first_token + it.page_end * P;  // exclusive
      const int lo = max(key_begin, W > 0 ? p - W + 1 : 0);
      const int hi = min(key_end - 1, p);

      bf16x8 qv[NKK];
      {
        // Unconditional loads (lanes past the block read its last head and
        // are zeroed), so they are in flight together.
        const uint16_t *qrow =
            a.q + (static_cast<size_t>(sd.q_start) * a.num_q_heads + it.kv_head * G + it.head0 + min(c16, nh - 1)) * D;
        if (sg.rope_off < 0) {
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            const u32x4 z = {0u, 0u, 0u, 0u};
            const u32x4 x = ld16(qrow + kk * 32 + u * 8);
            qv[kk] = as_bf16x8(c16 < nh ? x : z);
          }
        } else {
          relocate_row<D, NKK>(qv, qrow, 32, u * 8, c16 < nh, a.rope.tables + sg.rope_off, s_rope[wave], a.rope);
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
          const uint16_t *kpage = a.k_pool + static_cast<size_t>(page) * P * D;
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) {
            u32x4 x = {0u, 0u, 0u, 0u};
            if (ok) x = ld16(kpage + PL::k_elem(rel % P, 4 * kk + u));
            kb_[hb][kk] = x;
          }
        }
        const int key = kbase + 8 * u;
        const int rel = key - sg.first_token;
        const bool ok = key < key_end;
        const int page = P == 64 ? upage : (ok ? a.page_ids[sg.page_off + rel / P] : 0);
        const uint16_t *vpage = a.v_pool + static_cast<size_t>(page) * P * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
          u32x4 x = {0u, 0u, 0u, 0u};
          if (ok) x = ld16(vpage + PL::v_elem(db * 16 + c16, (rel % P) >> 3));
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
      const int nh = min(kDecodeCols, G - it.head0);
      const size_t out_row0 = static_cast<size_t>(sd.q_start) * a.num_q_heads + it.kv_head * G + it.head0;
      for (int e = tid; e < nh * TPC; e += kDecodeThreads) {
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

}  // namespace

hipError_t launch_decode(const DecodeArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s) {
  if (n_wgs <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(decode_kernel, head_dim, page_size, dim3(n_wgs), dim3(kDecodeThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs &a, int n_items, int max_entries, int head_dim, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  const int epp = 256 / (head_dim / 4);
  const dim3 grid(n_items, (max_entries + epp - 1) / epp);
  if (head_dim == 64) SEGKV_LAUNCH(combine_kernel<64>, grid, dim3(256), s, a);
  else if (head_dim == 128) SEGKV_LAUNCH(combine_kernel<128>, grid, dim3(256), s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
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

}  // namespace segkv
