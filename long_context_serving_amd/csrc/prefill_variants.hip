// HIP kernels of libsegkv: the prefill variants beside the default kernel
// (two groups one phase apart; four waves of 64 rows; software pipelined).

#include "kernels_common.h"
#include "page_layout.h"
#include "segkv_launch.h"

namespace segkv {
namespace {

// ===========================================================================
// Prefill, two-group schedule.  The eight waves form two groups of four with
// one wave of each group on every SIMD (waves w and w + 4 share a SIMD).  A
// wave takes each 64-key tile in two phases: a matrix phase (S^T = K Q^T of
// this tile, then O^T += V^T P^T of its previous tile) and a vector phase
// (mask, lazy online softmax, bf16 probabilities).  Group 1 runs one phase
// behind group 0 and a workgroup barrier ends every phase, so on each SIMD
// one wave's products run while the other wave's softmax runs: the matrix
// cores and the vector ALUs work side by side instead of in turn.
//
// Each workgroup walks a fixed list of work items, planned on the host
// (cost balanced over the resident workgroups), so the next item is always
// known: its tiles load ahead like any other tile, and its queries load
// during the last tile of the current item.  The output of an item is
// written in the vector phase after its last products.
//
// Group 0 issues every tile load into a four-stage LDS ring: tile g + 2
// starts loading when tile g's matrix phase begins (its stage was last read
// by group 1's products of tile g - 1), and tile g must be resident when
// that phase starts.  Group 1 issues no tile loads, so the waits the
// compiler places on its query loads cover nothing else.
// ===========================================================================
template <int D, int P>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_pp_kernel(PrefillArgs a) {
  using L = PrefillLds<D>;
  using PL = PageLayout<D, P>;
  constexpr int NKK = D / 16;  // k-steps of the QK product
  constexpr int NDB = D / 32;  // 32-channel blocks of O^T
  constexpr int NW = kPrefillThreads / 64;
  constexpr int PW = NW / 2;                                // producer waves (group 0)
  constexpr int K_INSTR = L::K_CHUNKS / (PW * 64);          // direct loads per producer lane per tile (K)
  constexpr int V_INSTR = L::V_CHUNKS / (PW * 64);          // (V^T)
  constexpr int LOADS_PER_TILE = K_INSTR + V_INSTR;
  constexpr int NR = 4;                                     // LDS ring stages
  static_assert(kPrefillRows == 32 * NW, "one 32-row column block per wave");
  static_assert(K_INSTR >= 1 && V_INSTR >= 1 && L::K_CHUNKS % (PW * 64) == 0 && L::V_CHUNKS % (PW * 64) == 0,
                "a tile is a whole number of loads per producer lane");
  __shared__ __attribute__((aligned(16))) uint4 smem4[NR * L::STAGE_BYTES / 16];
  __shared__ __attribute__((aligned(16))) float s_rope[NW][2 * D];  // per-wave relocation table
  char *smem = reinterpret_cast<char *>(smem4);
  static_assert(L::KCPR * 16 >= 128 && (L::KCPR * 16) % 128 == 0 && L::STAGE_BYTES % 256 == 0 &&
                    (L::K_CHUNKS * 16) % 256 == 0, "row starts leave the chunk bits free");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  // group 0: issues the tile loads, one phase ahead.  Taken from the first
  // lane so that every branch on it is a scalar branch: a wave must never
  // pass both arms of a boundary (each holds an s_barrier).
  const bool lead = __builtin_amdgcn_readfirstlane(wave) < PW;
  const int col = lane & 31, half = lane >> 5;
  const int G = a.group;
  const int rows = a.rows_per_tile;
  const int r = wave * 32 + col;  // this lane's row of an item
  const int pos_off = r / G;

  const int k_begin = sload(a.wg_items + blockIdx.x);
  const int k_end = sload(a.wg_items + blockIdx.x + 1);
  if (k_begin >= k_end) return;

  // ---- producer (group 0) -------------------------------------------------
  int p_k = k_begin, p_tile = 0, p_end = 0, issued = 0;  // next tile to issue; tiles issued so far
  SegDesc psg;
  auto p_set = [&](int idx) {
    const PrefillItem pi_ = sload(a.items + idx);
    p_tile = pi_.tile_begin;
    p_end = pi_.tile_end;
    psg = sload(a.segs + pi_.seq * a.num_kv_heads + pi_.kv_head);
  };
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
      const int c = (j * PW + wave) * 64 + lane;
      const int row = c / L::KCPR;
      const int logical = (c % L::KCPR) ^ L::k_swz(row);
      if constexpr (P == kTileKeys) {
        lds_dma16_s(a.k_pool + static_cast<size_t>(pid[0]) * (P * D), static_cast<uint32_t>(PL::k_elem(row, logical) * 2),
                    st + (j * PW + wave) * 1024);
      } else {
        int slot;
        const int page = page_of(row, &slot);
        lds_dma16(a.k_pool + static_cast<size_t>(page) * (P * D) + PL::k_elem(slot, logical), st + (j * PW + wave) * 1024);
      }
    }
#pragma unroll
    for (int j = 0; j < V_INSTR; ++j) {
      const int c = (j * PW + wave) * 64 + lane;
      const int d = c / 8;
      const int logical = (c % 8) ^ L::v_swz(d);
      if constexpr (P == kTileKeys) {
        lds_dma16_s(a.v_pool + static_cast<size_t>(pid[0]) * (P * D), static_cast<uint32_t>(PL::v_elem(d, logical) * 2),
                    st + L::K_CHUNKS * 16 + (j * PW + wave) * 1024);
      } else {
        int slot;
        const int page = page_of(logical * 8, &slot);
        lds_dma16(a.v_pool + static_cast<size_t>(page) * (P * D) + PL::v_elem(d, slot >> 3),
                  st + L::K_CHUNKS * 16 + (j * PW + wave) * 1024);
      }
    }
  };
  // Issue the workgroup's tiles in order until `upto` tiles are issued.
  auto produce = [&](int upto) {
    while (issued < upto && p_k < k_end) {
      issue_tile(p_tile, issued % NR);
      ++issued;
      // (>=: an item is never taken as holding fewer than one tile, so that
      // the producer and the tile loop below always agree and terminate)
      if (++p_tile >= p_end && ++p_k < k_end) p_set(p_k);
    }
  };
  // Phase boundary s; every wave passes the same boundaries 0, 1, 2, ...
  // Group 0's matrix phase of tile g starts after boundary 2g, group 1's
  // after 2g + 1.  At an even boundary group 0 first waits for its loads of
  // tile g (only tile g + 1's may stay in flight), and after the barrier it
  // starts tile g + 2, whose stage held tile g - 2: group 1 read that tile's
  // V^T last, before this barrier.
  auto boundary = [&](int s) {
    __builtin_amdgcn_sched_barrier(0);
    if (lead && (s & 1) == 0) {
      const int g = s >> 1;
      produce(g + 1);
      if (issued - (g + 1) >= 1)
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
      else
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
      produce(g + NR - 1);
    } else {
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // ---- rows of an item ----------------------------------------------------
  struct Rows {
    const uint16_t *qrow;  // query row read (an invalid row reads the item's last valid row)
    int h, t, p, vis_lo;   // query head, query index, key position, first visible key
    int p_wmin, p_wmax, W;  // wave-uniform: key positions of the wave's first and last rows; window
    bool valid;
  };
  auto rows_of = [&](const PrefillItem &x, const SeqDesc &sd, const SegDesc &sg) {
    Rows ri;
    ri.h = x.kv_head * G + (r - pos_off * G);
    const int t0 = x.qtile * rows;
    const int t_last = min(t0 + rows, sd.q_len) - 1;
    ri.t = t0 + pos_off;
    ri.valid = pos_off < rows && ri.t < sd.q_len;
    const int base = sd.kv_len - sd.q_len;
    ri.p = base + min(ri.t, t_last);
    ri.W = sg.window;
    ri.vis_lo = ri.W > 0 ? ri.p - ri.W + 1 : 0;
    // wave-uniform; read from the first lane so that the tile tests branch
    // on scalars
    ri.p_wmin = __builtin_amdgcn_readfirstlane(base + min(t0 + (wave * 32) / G, t_last));
    ri.p_wmax = __builtin_amdgcn_readfirstlane(base + min(t0 + (wave * 32 + 31) / G, t_last));
    ri.qrow = a.q + (static_cast<size_t>(sd.q_start + min(ri.t, t_last)) * a.num_q_heads + ri.h) * D;
    return ri;
  };

  bf16x8 qv[NKK];  // Q^T operand of the current item
  // Rows past the item's last query read that query's row: their scores are
  // finite and are never stored (each column is one row), so the loads need
  // no select and nothing waits for them before q_ready().
  auto load_q_plain = [&](const Rows &ri) {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) qv[kk] = as_bf16x8(ld16(ri.qrow + kk * 16 + half * 8));
  };
  auto load_q = [&](const Rows &ri, int rope_off) {
    if (rope_off < 0)
      load_q_plain(ri);
    else
      relocate_row<D, NKK, 1>(qv, ri.qrow, 16, half * 8, ri.valid, a.rope.tables + rope_off, s_rope[wave], a.rope);
  };
  // Makes the compiler wait for the query loads here (and not inside a
  // later phase, where its wait would also drain the tile loads).
  auto q_ready = [&]() {
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qv[kk]));
  };

  // Tile loads first: the first boundary waits for tile 0.
  if (lead) {
    p_set(k_begin);
    produce(2);
  }
  int k = k_begin;  // item whose tile the next step reads
  PrefillItem it = sload(a.items + k);
  SeqDesc sd = sload(a.seqs + it.seq);
  SegDesc sg = sload(a.segs + it.seq * a.num_kv_heads + it.kv_head);
  Rows qi = rows_of(it, sd, sg);
  load_q(qi, sg.rope_off);
  q_ready();

  // LDS byte offsets of this lane's operand chunks within a stage.  Chunk c
  // of a row sits at ((c ^ swizzle) << 4) from the row start, and the row
  // starts are multiples of 128 bytes, so chunk 2 j + half of the lane's row
  // is at lane_off ^ (j << 5): one XOR per read, with no per-read register
  // kept across the loop.
  const int key_a0 = st_row_key(col);  // K row this lane feeds to block 0 (block 1: +32)
  const int k_lane = key_a0 * L::KCPR * 16 + ((half ^ L::k_swz(key_a0)) << 4);
  const int v_lane = L::K_CHUNKS * 16 + col * 128 + ((half ^ L::v_swz(col)) << 4);  // V^T row db*32 + col: + db*4096

  f32x16 oacc[NDB];
#pragma unroll
  for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
  float m = kNegInf;  // running (lazy) max of raw scores of this column
  float l = 0.f;      // this lane's share of the running sum
  bf16x8 pb[4];       // probabilities of the previous step's tile
  bool have_p = false;
  int p_stage = 0;
  // Output rows of the item being accumulated, written once its last
  // products are done (flush).
  bool flush = false;
  int o_part = -1, o_h = 0, o_t = 0, o_qs = 0;
  bool o_valid = false;

  // S^T = K Q^T for one tile.  Operand reads run kLookahead products ahead
  // of the products through a small register ring.
  constexpr int kLookahead = 4;
  auto qk = [&](int st_off, f32x16 &s0, f32x16 &s1) {
    s0 = f32x16{};
    s1 = f32x16{};
    constexpr int N = 2 * NKK;  // products: (k-step kk, key block b) at i = 2 kk + b
    const int kb = st_off + k_lane;
    bf16x8 kr[kLookahead];
    auto kread = [&](int i) {
      kr[i % kLookahead] =
          as_bf16x8(*reinterpret_cast<const u32x4 *>(smem + (kb ^ ((i >> 1) << 5)) + (i & 1) * 32 * L::KCPR * 16));
    };
#pragma unroll
    for (int i = 0; i < kLookahead; ++i) kread(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      if (i & 1)
        s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % kLookahead], qv[i >> 1], s1, 0, 0, 0);
      else
        s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % kLookahead], qv[i >> 1], s0, 0, 0, 0);
      if (i + kLookahead < N) kread(i + kLookahead);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // O^T += V^T P^T for the previous step's tile.
  auto pv = [&](int st_off) {
    constexpr int N = 4 * NDB;  // products: (16-key step, channel block db) at i = step * NDB + db
    const int vb = st_off + v_lane;
    bf16x8 va[kLookahead];
    auto vread = [&](int i) {
      va[i % kLookahead] =
          as_bf16x8(*reinterpret_cast<const u32x4 *>(smem + (vb ^ ((i / NDB) << 5)) + (i % NDB) * 32 * 128));
    };
#pragma unroll
    for (int i = 0; i < kLookahead; ++i) vread(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      __builtin_amdgcn_sched_barrier(0);
      oacc[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % kLookahead], pb[i / NDB], oacc[i % NDB], 0, 0, 0);
      if (i + kLookahead < N) vread(i + kLookahead);
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Scores of keys this row cannot see become -inf (tiles on the causal
  // diagonal or a window edge only).
  auto mask = [&](f32x16 &s0, f32x16 &s1, int k0, const Rows &ri) {
    // key = k0 + 16 (v/8) + 8 half + v%8 (+32 for block 1); visible iff
    // vis_lo <= key <= p, tested as one unsigned range compare.
    const unsigned lo_rel = static_cast<unsigned>(ri.vis_lo - k0 - 8 * half);
    const unsigned span = static_cast<unsigned>(ri.p - ri.vis_lo);
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int off = ((v >> 3) << 4) + (v & 7);
      if (static_cast<unsigned>(off) - lo_rel > span) s0[v] = kNegInf;
      if (static_cast<unsigned>(off + 32) - lo_rel > span) s1[v] = kNegInf;
    }
  };
  // Lazy online softmax and bf16 probabilities of the current tile.
  auto softmax = [&](f32x16 &s0, f32x16 &s1) {
    float mx = max32(s0, s1);
    {
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // Lazy running max (the lane pair of a column takes the same decision).
    const bool bump = mx * a.scale_log2 > m * a.scale_log2 + kRescaleLog2;
    const float m_new = bump ? mx : m;
    const float msc = m_new == kNegInf ? 0.f : m_new * a.scale_log2;
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
    // pb[2 kb + s] holds keys 32 kb + 16 s .. +15 of the tile (PV k-step 2 kb + s)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const f32x16 &sv = kb ? s1 : s0;
        pb[2 * kb + s] = pack8_bf16(sv[8 * s + 0], sv[8 * s + 1], sv[8 * s + 2], sv[8 * s + 3], sv[8 * s + 4],
                                    sv[8 * s + 5], sv[8 * s + 6], sv[8 * s + 7]);
      }
  };
  // Output of the finished item: normalised rows (or fp32 partials) and LSE.
  auto write_out = [&]() {
    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_val = l_tot > 0.f ? m * a.scale + logf(l_tot) : kNegInf;
    if (o_part < 0) {
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
          for (int kx = 0; kx < 2; ++kx) {
            // lanes 32-63 of the first operand trade with lanes 0-31 of the second
            const auto sw = __builtin_amdgcn_permlane32_swap(p0[kx], p1[kx], false, false);
            w[db][ip][kx] = sw[0];
            w[db][ip][2 + kx] = sw[1];
          }
        }
      }
      if (o_valid) {
        uint16_t *orow = a.o + (static_cast<size_t>(o_qs + o_t) * a.num_q_heads + o_h) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int ip = 0; ip < 2; ++ip) *reinterpret_cast<u32x4 *>(orow + db * 32 + ip * 16 + half * 8) = w[db][ip];
        if (half == 0 && a.lse) a.lse[static_cast<size_t>(o_qs + o_t) * a.num_q_heads + o_h] = lse_val;
      }
    } else {
      float *prow = a.part_o + (static_cast<size_t>(o_part) * kPrefillRows + r) * D;
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
      if (half == 0) a.part_lse[static_cast<size_t>(o_part) * kPrefillRows + r] = lse_val;
    }
  };

  int tile = it.tile_begin;
  int s = 0;
  if (!lead) boundary(s++);  // group 1 starts one phase later
  for (int g = 0;; ++g) {
    const bool done = k >= k_end;  // only the last tile's products and the output remain
    boundary(s++);
    // ---- matrix phase: S^T of tile g, then O^T of tile g - 1 ----
    const int k0 = tile * kTileKeys;
    const bool empty = done || k0 > qi.p_wmax || (qi.W > 0 && k0 + kTileKeys - 1 < qi.p_wmin - qi.W + 1);
    const bool full = k0 + kTileKeys - 1 <= qi.p_wmin && (qi.W == 0 || k0 >= qi.p_wmax - qi.W + 1);
    const bool last_tile = !done && tile + 1 >= it.tile_end;
    const bool next = last_tile && k + 1 < k_end;
    PrefillItem nit;  // descriptors of item k + 1, read at its last tile
    SeqDesc nsd;
    SegDesc nsg;
    if (next) {
      nit = sload(a.items + k + 1);
      nsd = sload(a.seqs + nit.seq);
      nsg = sload(a.segs + nit.seq * a.num_kv_heads + nit.kv_head);
    }
    f32x16 s0, s1;  // scores of tile g (defined when the tile is not empty for this wave)
    if (!empty) qk((g % NR) * L::STAGE_BYTES, s0, s1);
    if (next && nsg.rope_off < 0) load_q_plain(rows_of(nit, nsd, nsg));  // the next item's queries
    if (have_p) pv(p_stage * L::STAGE_BYTES);
    boundary(s++);
    // ---- vector phase ----
    if (flush) {
      write_out();
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
      m = kNegInf;
      l = 0.f;
      flush = false;
    }
    if (done) break;
    have_p = !empty;
    if (!empty) {
      p_stage = g % NR;
      if (!full) mask(s0, s1, k0, qi);
      softmax(s0, s1);
    }
    if (last_tile) {
      flush = true;
      o_part = it.part;
      o_h = qi.h;
      o_t = qi.t;
      o_qs = sd.q_start;
      o_valid = qi.valid;
      ++k;
      if (next) {
        it = nit;
        sd = nsd;
        sg = nsg;
        qi = rows_of(it, sd, sg);
        if (sg.rope_off >= 0) load_q(qi, sg.rope_off);
        q_ready();
        tile = it.tile_begin;
      }
    } else {
      ++tile;
    }
  }
  if (lead) boundary(s++);  // the boundary group 1 passed before its last phase
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
  using PL = PageLayout<D, P>;
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
        src = a.k_pool + static_cast<size_t>(pid[0]) * (P * D) + PL::k_elem(row, logical);
      } else {
        int slot;
        const int page = page_of(row, &slot);
        src = a.k_pool + static_cast<size_t>(page) * (P * D) + PL::k_elem(slot, logical);
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
        src = a.v_pool + static_cast<size_t>(pid[0]) * (P * D) + PL::v_elem(d, logical);
      } else {
        int slot;
        const int page = page_of(logical * 8, &slot);
        src = a.v_pool + static_cast<size_t>(page) * (P * D) + PL::v_elem(d, slot >> 3);
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
        // Empty asm statements pin the program order (the product pair, then
        // the body slice under it): the body's pure arithmetic would
        // otherwise be hoisted above all the products of the step.
        asm volatile("" : "+v"(vf));
#pragma unroll
        for (int c = 0; c < 2; ++c)
          oacc[c][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, (*pk_prev)[c][ks], oacc[c][db], 0, 0, 0);
        const int j0 = g * VPG;
        body(pk_cur, j0 / 16, j0 % 16, VPG);
        asm volatile("" : "+v"(l[j0 / 16]));
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
// Prefill, software pipelined (SEGKV_TUNE_PREFILL_KERNEL = 4).  The same
// work items, queue, tile loads and output as prefill_kernel, with the tile
// loop of each item reordered so that every wave has independent vector
// work to issue while its own products run:
//
//   step c:  S^T(c+1) = K(c+1) Q^T      beside   exp / row sum / pack of tile c
//            O^T += V^T(c) P^T(c)        beside   mask / max of tile c+1
//            rescale for tile c+1 (when its max moved), then the tile barrier
//
// (the first tile's product is issued before the item's first step, the
// last step has no next tile).  A step reads K of tile c+1 and V^T of tile
// c, so the LDS ring has four stages and the barrier that ends step c waits
// for tile c+2; tile c+4 starts loading right after it, into the stage tile
// c used.  The products and the vector work of a step sit in one basic
// block, and scheduling group barriers ask the compiler to alternate them.
// ===========================================================================
template <int D, int P>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_sp_kernel(PrefillArgs a) {
  using L = PrefillLds<D>;
  using PL = PageLayout<D, P>;
  constexpr int NKK = D / 16;  // k-steps of the QK product
  constexpr int NDB = D / 32;  // 32-channel blocks of O^T
  constexpr int NW = kPrefillThreads / 64;
  constexpr int K_INSTR = L::K_CHUNKS / kPrefillThreads;  // direct loads per lane per tile (K)
  constexpr int V_INSTR = L::V_CHUNKS / kPrefillThreads;  // (V^T)
  constexpr int NSTAGE = 4;
  constexpr int LOADS_PER_TILE = K_INSTR + V_INSTR;
  static_assert(kPrefillRows == 32 * NW, "one 32-row column block per wave");
  static_assert(K_INSTR >= 1 && V_INSTR >= 1, "tile smaller than one load per lane");
  static_assert(L::KCPR * 16 >= 128 && (L::KCPR * 16) % 128 == 0 && L::STAGE_BYTES % 256 == 0 &&
                    (L::K_CHUNKS * 16) % 256 == 0, "row starts leave the chunk bits free");
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

  if (tid == 0) s_next[0] = atomicAdd(a.counter, 1);
  __syncthreads();
  int cur = __builtin_amdgcn_readfirstlane(s_next[0]);
  if (cur >= n_items) return;
  int nxt = -1;
  int fslot = 1;

  // ---- producer: global->LDS tile loads, across item boundaries ----------
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
  int issued = 0, consumed = 0;  // tiles issued / steps finished so far (the stream of the workgroup's tiles)
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
      if constexpr (P == kTileKeys) {
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
      if (++p_tile >= p_end) {
        if (p_item == cur && nxt >= 0 && nxt < n_items)
          p_set(nxt);
        else
          p_item = -1;  // resumes once the consumer knows the item after this one
      }
    }
  };
  // Workgroup barrier that leaves the newest `pending` issued tiles' loads
  // in flight (this wave's LDS operations and older tile loads complete
  // first).
  auto sync_tiles = [&](int pending) {
    if (pending >= 2)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(2 * LOADS_PER_TILE) : "memory");
    else if (pending == 1)
      asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(LOADS_PER_TILE) : "memory");
    else
      asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
  };
  // Make tiles [0, need) of the stream resident: issue what is missing and
  // wait, leaving later tiles in flight.  `ready` counts the tiles known
  // resident (all waves take the same decisions: the counts are uniform).
  int ready = 0;
  auto ensure = [&](int need) {
    if (issued < need) produce(need);
    sync_tiles(issued - need);
    ready = min(need, issued);
  };

  produce(3);
  ensure(2);

  // LDS byte offsets of this lane's operand chunks within a stage: chunk
  // 2 j + half of the lane's row sits at lane_off ^ (j << 5).
  const int key_a0 = st_row_key(col);  // K row this lane feeds to block 0 (block 1: +32)
  const int k_lane = key_a0 * L::KCPR * 16 + ((half ^ L::k_swz(key_a0)) << 4);
  const int v_lane = L::K_CHUNKS * 16 + col * 128 + ((half ^ L::v_swz(col)) << 4);

  while (true) {
    const PrefillItem it = sload(a.items + cur);
    const SeqDesc sd = sload(a.seqs + it.seq);
    const SegDesc sg = sload(a.segs + it.seq * a.num_kv_heads + it.kv_head);
    const int h = it.kv_head * G + (r - pos_off * G);
    const int t0 = it.qtile * rows;
    const int t_last = min(t0 + rows, sd.q_len) - 1;
    const int t = t0 + pos_off;
    const bool valid = pos_off < rows && t < sd.q_len;
    const int base = sd.kv_len - sd.q_len;
    const int p = base + min(t, t_last);
    const int W = sg.window;
    const int vis_lo = W > 0 ? p - W + 1 : 0;
    const int p_wmin = __builtin_amdgcn_readfirstlane(base + min(t0 + (wave * 32) / G, t_last));
    const int p_wmax = __builtin_amdgcn_readfirstlane(base + min(t0 + (wave * 32 + 31) / G, t_last));

    bf16x8 qv[NKK];
    {
      const uint16_t *qrow = a.q + (static_cast<size_t>(sd.q_start + min(t, t_last)) * a.num_q_heads + h) * D;
      if (sg.rope_off < 0) {
#pragma unroll
        for (int kk = 0; kk < NKK; ++kk) qv[kk] = as_bf16x8(ld16(qrow + kk * 16 + half * 8));
      } else {
        relocate_row<D, NKK>(qv, qrow, 16, half * 8, valid, a.rope.tables + sg.rope_off, s_rope[wave], a.rope);
      }
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) asm volatile("" : "+v"(qv[kk]));
    }

    f32x16 oacc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) oacc[db] = f32x16{};
    float m = kNegInf;  // running (lazy) max of raw scores of this column
    float msc = 0.f;    // m * scale_log2 (0 while m is -inf)
    float l = 0.f;      // this lane's share of the running sum

    // per-wave tile class: 0 empty, 1 edge (per-key mask), 2 full
    auto tile_class = [&](int tile) {
      const int k0 = tile * kTileKeys;
      const bool empty = k0 > p_wmax || (W > 0 && k0 + kTileKeys - 1 < p_wmin - W + 1);
      const bool full = k0 + kTileKeys - 1 <= p_wmin && (W == 0 || k0 >= p_wmax - W + 1);
      return empty ? 0 : (full ? 2 : 1);
    };
    // QK product of one tile into (s0, s1); K operand reads run four
    // products ahead.
    auto qk = [&](int st_off, f32x16 &s0, f32x16 &s1) {
      s0 = f32x16{};
      s1 = f32x16{};
      constexpr int N = 2 * NKK;
      constexpr int LA = 4;
      const int kb = st_off + k_lane;
      bf16x8 kr[LA];
      auto kread = [&](int i) {
        kr[i % LA] = as_bf16x8(*reinterpret_cast<const u32x4 *>(smem + (kb ^ ((i >> 1) << 5)) + (i & 1) * 32 * L::KCPR * 16));
      };
#pragma unroll
      for (int i = 0; i < LA; ++i) kread(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        if (i & 1)
          s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % LA], qv[i >> 1], s1, 0, 0, 0);
        else
          s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[i % LA], qv[i >> 1], s0, 0, 0, 0);
        if (i + LA < N) kread(i + LA);
      }
    };
    // PV product of one tile from pb; V^T operand reads run four products ahead.
    auto pv = [&](int st_off, const bf16x8 (&pb)[4]) {
      constexpr int N = 4 * NDB;
      constexpr int LA = 4;
      const int vb = st_off + v_lane;
      bf16x8 va[LA];
      auto vread = [&](int i) {
        va[i % LA] = as_bf16x8(*reinterpret_cast<const u32x4 *>(smem + (vb ^ ((i / NDB) << 5)) + (i % NDB) * 32 * 128));
      };
#pragma unroll
      for (int i = 0; i < LA; ++i) vread(i);
#pragma unroll
      for (int i = 0; i < N; ++i) {
        oacc[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[i % LA], pb[i / NDB], oacc[i % NDB], 0, 0, 0);
        if (i + LA < N) vread(i + LA);
      }
    };
    auto mask = [&](f32x16 &s0, f32x16 &s1, int k0) {
      const unsigned lo_rel = static_cast<unsigned>(vis_lo - k0 - 8 * half);
      const unsigned span = static_cast<unsigned>(p - vis_lo);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int off = ((v >> 3) << 4) + (v & 7);
        if (static_cast<unsigned>(off) - lo_rel > span) s0[v] = kNegInf;
        if (static_cast<unsigned>(off + 32) - lo_rel > span) s1[v] = kNegInf;
      }
    };
    // Row max of a tile (both lanes of a column).
    auto tile_max = [&](const f32x16 &s0, const f32x16 &s1) {
      float mx = max32(s0, s1);
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
      return fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    };
    // Lazy running max: move it (and rescale O and l) only when the tile's
    // max exceeds it by more than 2^kRescaleLog2.
    auto update_max = [&](float mx) {
      const bool bump = mx * a.scale_log2 > m * a.scale_log2 + kRescaleLog2;
      const float m_new = bump ? mx : m;
      const float msc_new = m_new == kNegInf ? 0.f : m_new * a.scale_log2;
      if (__builtin_expect(__builtin_amdgcn_ballot_w64(bump) != 0, 0)) {
        const float alpha = bump ? fast_exp2(m * a.scale_log2 - msc_new) : 1.f;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) oacc[db] *= alpha;
      }
      m = m_new;
      msc = msc_new;
    };
    // exp, row sum and bf16 probabilities of a tile (scores in place).
    auto probs = [&](f32x16 &s0, f32x16 &s1, bf16x8 (&pb)[4]) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s0[v] = fast_exp2(fmaf(s0[v], a.scale_log2, -msc));
        s1[v] = fast_exp2(fmaf(s1[v], a.scale_log2, -msc));
      }
      l += sum32(s0, s1);
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const f32x16 &sv = kb ? s1 : s0;
          pb[2 * kb + s] = pack8_bf16(sv[8 * s + 0], sv[8 * s + 1], sv[8 * s + 2], sv[8 * s + 3], sv[8 * s + 4],
                                      sv[8 * s + 5], sv[8 * s + 6], sv[8 * s + 7]);
        }
    };

    const int fetch_tile = max(it.tile_begin, it.tile_end - 4);
    // The item's first two tiles may have been issued only after the last
    // wait (short items: the next item's index arrives late).
    {
      const int need = consumed + min(2, it.tile_end - it.tile_begin);
      if (ready < need) ensure(need);
    }
    // Scores of the tile the next step takes.  Tiles a wave's rows cannot see
    // at all are computed like edge tiles (every score masked to -inf, so
    // they add nothing): the step stays one block of code.
    f32x16 sc0, sc1;
    {
      qk((consumed % NSTAGE) * L::STAGE_BYTES, sc0, sc1);
      if (tile_class(it.tile_begin) != 2) mask(sc0, sc1, it.tile_begin * kTileKeys);
      update_max(tile_max(sc0, sc1));
    }
    // After a step: wait for tile c + 2 of the stream (the next step reads
    // tile c + 1's V^T and tile c + 2's K), then refill the freed stage.
    auto end_step = [&](int tile) {
      ensure(consumed + 3);
      ++consumed;
      if (tile == fetch_tile) {
        nxt = __builtin_amdgcn_readfirstlane(s_next[fslot]);
        fslot ^= 1;
        if (p_item < 0 && nxt < n_items) p_set(nxt);
      }
      produce(consumed + NSTAGE);
      // a step may read the item's next tile only once it is resident
      if (tile + 2 < it.tile_end && ready < consumed + 2) ensure(consumed + 2);
    };
    for (int tile = it.tile_begin; tile + 1 < it.tile_end; ++tile) {
      if (tile == fetch_tile && tid == 0) s_next[fslot] = atomicAdd(a.counter, 1);
      const int st_c = (consumed % NSTAGE) * L::STAGE_BYTES;
      const int st_n = ((consumed + 1) % NSTAGE) * L::STAGE_BYTES;
      f32x16 sn0, sn1;
      bf16x8 pb[4];
      qk(st_n, sn0, sn1);
      probs(sc0, sc1, pb);
#pragma unroll
      for (int i = 0; i < 2 * NKK; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);  // six VALU
      }
      pv(st_c, pb);
      if (tile_class(tile + 1) != 2) mask(sn0, sn1, (tile + 1) * kTileKeys);
      const float mx = tile_max(sn0, sn1);
#pragma unroll
      for (int i = 0; i < 4 * NDB; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 1);
      }
      update_max(mx);
      sc0 = sn0;
      sc1 = sn1;
      end_step(tile);
    }
    {
      const int tile = it.tile_end - 1;
      if (tile == fetch_tile && tid == 0) s_next[fslot] = atomicAdd(a.counter, 1);
      bf16x8 pb[4];
      probs(sc0, sc1, pb);
      pv((consumed % NSTAGE) * L::STAGE_BYTES, pb);
      end_step(tile);
    }

    const float l_tot = l + __shfl_xor(l, 32);
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    const float lse_val = l_tot > 0.f ? m * a.scale + logf(l_tot) : kNegInf;
    if (it.part < 0) {
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

    if (nxt >= n_items) break;
    cur = nxt;
    nxt = -1;
  }
}

// ===========================================================================
// Two workgroups per CU (tuning value 5): the default kernel's schedule and
// layout with 4 waves of 32 rows per workgroup, 128 rows per work item and
// two resident workgroups, each with its own item queue position, barriers
// and two K/V stages.  One workgroup's item starts and ends then overlap the
// other's tiles, and the waves sharing a SIMD belong to different
// workgroups, which do not meet at barriers.
// ===========================================================================

template <int D, int P>
__global__ __launch_bounds__(kPrefillDuoThreads, 2) void prefill_duo_kernel(PrefillArgs a) {
  using L = PrefillLds<D>;
  using PL = PageLayout<D, P>;
  constexpr int NKK = D / 16;  // k-steps of the QK product
  constexpr int NDB = D / 32;  // 32-channel blocks of O^T
  constexpr int NW = kPrefillDuoThreads / 64;
  constexpr int K_INSTR = L::K_CHUNKS / kPrefillDuoThreads;  // direct loads per lane per tile (K)
  constexpr int V_INSTR = L::V_CHUNKS / kPrefillDuoThreads;  // (V^T)
  constexpr int NSTAGE = 2;  // two workgroups of two stages each fit a CU's LDS
  constexpr int LOADS_PER_TILE = K_INSTR + V_INSTR;
  static_assert(kPrefillDuoRows == 32 * NW && kPrefillDuoRows <= kPrefillRows,
                "one 32-row column block per wave; an item's rows fit a partial slot");
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
      produce(consumed + NSTAGE);
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

hipError_t launch_prefill_sp(const PrefillArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s) {
  if (n_wgs <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(prefill_sp_kernel, head_dim, page_size, dim3(n_wgs), dim3(kPrefillThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_pp(const PrefillArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s) {
  if (n_wgs <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(prefill_pp_kernel, head_dim, page_size, dim3(n_wgs), dim3(kPrefillThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_wide(const PrefillArgs &a, int n_items, int head_dim, int page_size, hipStream_t s) {
  if (n_items <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(prefill_wide_kernel, head_dim, page_size, dim3(n_items), dim3(kPrefillWideThreads), s, a);
  return hipGetLastError();
}

hipError_t launch_prefill_duo(const PrefillArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s) {
  if (n_wgs <= 0) return hipSuccess;
  SEGKV_DISPATCH_DP(prefill_duo_kernel, head_dim, page_size, dim3(n_wgs), dim3(kPrefillDuoThreads), s, a);
  return hipGetLastError();
}

}  // namespace segkv
