// HIP kernel of libsegkv: varlen prefill attention (8 waves x 32 rows, the default).

#include "kernels_common.h"
#include "page_layout.h"
#include "segkv_launch.h"

namespace segkv {
namespace {

// ===========================================================================
// Prefill: a persistent grid, one workgroup per CU.  Each workgroup takes
// work items from a queue in list order (longest first); an item is 256
// (query position, query head) rows of one (sequence, KV head group) over a
// range of 64-key tiles.  The K/V tile loads run two tiles ahead across item
// boundaries, so a workgroup never waits for its next item's first tiles.
// The MFMA operand layout and the LDS tile layout are described in
// kernels_common.h.
// ===========================================================================

template <int D, int P>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_kernel(PrefillArgs a) {
  using L = PrefillLds<D>;
  using PL = PageLayout<D, P>;
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
        lds_dma16_s(a.k_pool + static_cast<size_t>(pid[0]) * (P * D), static_cast<uint32_t>(PL::k_elem(row, logical) * 2),
                    st + (j * NW + wave) * 1024);
      } else {
        int slot;
        const int page = page_of(row, &slot);
        lds_dma16(a.k_pool + static_cast<size_t>(page) * (P * D) + PL::k_elem(slot, logical), st + (j * NW + wave) * 1024);
      }
    }
#pragma unroll
    for (int j = 0; j < V_INSTR; ++j) {
      const int c = (j * NW + wave) * 64 + lane;
      const int d = c / 8;
      const int logical = (c % 8) ^ L::v_swz(d);
      if constexpr (P == kTileKeys) {
        lds_dma16_s(a.v_pool + static_cast<size_t>(pid[0]) * (P * D), static_cast<uint32_t>(PL::v_elem(d, logical) * 2),
                    st + L::K_CHUNKS * 16 + (j * NW + wave) * 1024);
      } else {
        int slot;
        const int page = page_of(logical * 8, &slot);
        lds_dma16(a.v_pool + static_cast<size_t>(page) * (P * D) + PL::v_elem(d, slot >> 3),
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

}  // namespace

hipError_t launch_prefill(const PrefillArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(prefill_kernel, head_dim, page_size, dim3(n_items), dim3(kPrefillThreads), s, a);
  return hipGetLastError();
}

}  // namespace segkv
