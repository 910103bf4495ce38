// Internal layout shared by the host library and its HIP kernels.
//
// Device tables are rebuilt on the host for every call and copied from
// pinned staging to the start of the call's device workspace (caller-owned,
// or the fixed scratch of segkv_decode_noalloc), in this order:
//   SeqDesc  [n_seqs]
//   SegDesc  [n_seqs * num_kv_heads]
//   int32    page ids of every listed segment (SegDesc::page_off indexes here)
//   float    relocation tables, 2 * head_dim floats per distinct nonzero
//            offset of the listed segments (SegDesc::rope_off indexes here)
//   work items of the call (ScatterItem, PrefillItem or DecodeItem)
//   combine items (CombineItem), when the call has split work
// Split partials follow the tables at the next 256-byte boundary.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace segkv {

constexpr int kTileKeys = 64;      // keys per prefill KV tile (one LDS stage)
constexpr int kPrefillRows = 256;  // (query position, query head) rows per prefill workgroup
constexpr int kPrefillThreads = 512;  // 8 waves, 32 rows each, two per SIMD
constexpr int kPrefillWideThreads = 256;  // wide variant: 4 waves, 64 rows each, one per SIMD
constexpr int kDecodeThreads = 512;  // 8 waves, two per SIMD
constexpr int kDecodeCols = 16;    // query heads handled by one decode work item (a block of the GQA group, padded)
constexpr int kDecodeSlots = 16;   // LDS partials of one decode workgroup: (piece, wave) pairs of a batch
constexpr int kScatterThreads = 256;
constexpr int kScatterCopyWgs = 16;  // most workgroups of a scatter launch that copy staged tables
constexpr int kMergeThreads = 256;
constexpr int kTopkThreads = 1024;
constexpr int kTopkRun = 8;  // consecutive keys per thread per batch
constexpr int kMergeUnroll = 4;    // (row, head) pairs in flight per lane of the merge kernel
constexpr int kPrefillWgPerCu = 1;  // resident prefill workgroups per CU (104 KiB of LDS each at D = 128): the persistent grid
constexpr int kScoreWgPerCu = 2;  // resident token-score workgroups per CU (4 waves of 64 rows each)
constexpr int kScorePiecesPerSlot = 2;  // automatic token-score pieces: about this many per resident workgroup
constexpr int kDecodeWgPerCu = 1;   // resident decode workgroups per CU (the stream-K grid size)
constexpr int kXcds = 8;           // MI355X: workgroup i of a launch runs on XCD i % 8

struct SeqDesc {
  int32_t kv_len;   // tokens in the sequence (this layer)
  int32_t q_start;  // first row of this sequence in q / o
  int32_t q_len;    // queries (the last q_len tokens)
  int32_t pad;
};

struct SegDesc {
  int32_t first_token;  // logical index of the first token on page 0 (multiple of page_size)
  int32_t page_off;     // index of page 0 in the page id table
  int32_t n_pages;
  int32_t window;       // 0 = global, W >= 1 = local
  int32_t rope_off;     // -1: queries used as given; else the segment's relocation table
                        // (cos[head_dim], then signed sin[head_dim]) starts at float rope_off
  int32_t pad0, pad1, pad2;
};

// Query relocation: channel c of a relocated query becomes
// cos[c] * q[c] + ssin[c] * q[partner(c)], where channels below `lo` have
// cos 1 and ssin 0 and, above it, partner(c) = c +- half (style 0) or c ^ 1
// (style 1).  lo and half are multiples of 8, so a 16-byte chunk of
// channels has its partners in one chunk.
struct RopeArgs {
  const float *tables;
  int32_t lo;     // first rotary channel
  int32_t half;   // rotary channels / 2
  int32_t style;  // 0 rotate-half, 1 interleaved
  int32_t pad;
};

// One page touched by an append: K rows [slot_begin, slot_end) come from
// new-token rows src_row ..; when zero_tail is set the page is new and slots
// [slot_end, page_size) are cleared so that no live page holds stale bits.
// copy_from >= 0: the page replaces a page shared with a fork, whose slots
// [0, slot_begin) are copied first (copy-on-write).
struct ScatterItem {
  int32_t page_id;
  int32_t kv_head;
  int32_t slot_begin;
  int32_t slot_end;
  int32_t src_row;
  int32_t zero_tail;
  int32_t copy_from;
  int32_t pad1;
};

// One prefill work item: rows [qtile*rows_per_tile ...) of (sequence, KV head
// group) over KV tiles [tile_begin, tile_end).  part >= 0 writes fp32
// partial results to partial slot `part` instead of the final output.
struct PrefillItem {
  int32_t seq;
  int32_t kv_head;
  int32_t qtile;
  int32_t tile_begin;
  int32_t tile_end;
  int32_t part;
  int32_t pad0, pad1;
};

// One decode piece: pages [page_begin, page_end) of segment (seq, kv_head).
// The segment is covered by n_parts pieces (partial slots [part_begin,
// part_begin + n_parts)); with n_parts == 1 the piece writes the output,
// otherwise its partial goes to slot `part`.
struct DecodeItem {
  int32_t seq;
  int32_t kv_head;
  int32_t page_begin;
  int32_t page_end;
  int32_t part;
  int32_t part_begin;
  int32_t n_parts;
  int32_t head0;  // first query head of the item's block within the KV group (a multiple of kDecodeCols)
};

// One combine workgroup: merge partial slots [part_begin, part_begin+n_parts)
// for `rows` output rows starting at row `out_row` (row = query token), each
// row holding `heads` query heads starting at head `head0`.
struct CombineItem {
  int32_t part_begin;
  int32_t n_parts;
  int32_t out_row;
  int32_t rows;
  int32_t head0;
  int32_t heads;
  int32_t pad0, pad1;
};

// Workgroups [0, copy_wgs) of a scatter launch copy copy_n16 16-byte words
// from copy_src (pinned host memory) to copy_dst: the tables of the prefill
// that follows the append.  The scatter items go to workgroups copy_wgs ..
struct ScatterArgs {
  const uint16_t *k_new;
  const uint16_t *v_new;
  uint16_t *k_pool;
  uint16_t *v_pool;
  const ScatterItem *items;
  const uint4 *copy_src;
  uint4 *copy_dst;
  int32_t copy_n16;
  int32_t copy_wgs;
  int32_t num_kv_heads;
};

struct PrefillArgs {
  const uint16_t *q;
  uint16_t *o;
  float *lse;
  const uint16_t *k_pool;
  const uint16_t *v_pool;
  const SeqDesc *seqs;
  const SegDesc *segs;
  const int32_t *page_ids;
  const PrefillItem *items;
  float *part_o;    // [parts][kPrefillRows][head_dim] fp32, normalised
  float *part_lse;  // [parts][kPrefillRows] natural log
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;          // num_q_heads / num_kv_heads
  int32_t rows_per_tile;  // query positions per workgroup = kPrefillRows / group
  float scale_log2;       // softmax scale * log2(e)
  float scale;
  RopeArgs rope;
  int32_t n_items;        // work items; workgroups take them in list order from *counter
  int32_t *counter;       // zero at launch (part of the uploaded tables)
  const int32_t *wg_items;  // two-group kernel: workgroup w runs items [wg_items[w], wg_items[w + 1])
};

struct DecodeArgs {
  const uint16_t *q;
  const uint16_t *k_pool;
  const uint16_t *v_pool;
  const SeqDesc *seqs;
  const SegDesc *segs;
  const int32_t *page_ids;
  const DecodeItem *items;     // pieces, grouped by workgroup
  const int32_t *wg_piece_off; // [n_wgs + 1]: workgroup w runs pieces [off[w], off[w+1])
  float *part_o;    // [parts][kDecodeCols][head_dim]
  float *part_lse;  // [parts][kDecodeCols]
  uint16_t *o;        // [n_seqs][num_q_heads][head_dim]
  float *lse;         // [n_seqs][num_q_heads] or null
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  float scale_log2;
  float scale;
  RopeArgs rope;
};

// Partial slot layout for combine: slot s holds `slot_rows` rows of
// head_dim fp32 values and slot_rows lse values; row r of a slot maps to
// output (token row out_row + r / heads, head head0 + r % heads).
struct CombineArgs {
  const float *part_o;
  const float *part_lse;
  const CombineItem *items;
  uint16_t *o;
  float *lse;
  int32_t num_q_heads;
  int32_t slot_rows;
};

// Attention-mass token scores.  Work items are PrefillItems over the tiles
// of the query chunk; PrefillItem::part is the item's first partial row (one
// row = the 64 key sums of one tile).
struct ScoreArgs {
  const uint16_t *q;
  const float *lse;      // [sum q][num_q_heads], natural log, from the prefill of the same queries
  const uint16_t *k_pool;
  const SeqDesc *seqs;
  const SegDesc *segs;
  const int32_t *page_ids;
  const PrefillItem *items;
  int32_t *counter;      // work queue: items taken past the grid's first ones (0 at launch)
  int32_t n_items;
  float *part;           // [partial rows][64]
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;
  int32_t rows_per_tile;
  float scale_log2;
  RopeArgs rope;
};

// One 64-key tile of one sequence's chunk: its key sums are the partial rows
// part_idx[begin .. end), added in an order fixed by their positions there.
struct ScoreRow {
  int32_t seq;
  int32_t tile;
  int32_t begin;
  int32_t end;
};

struct ScoreReduceArgs {
  const float *part;
  const int32_t *part_idx;
  const ScoreRow *rows;
  const SeqDesc *seqs;
  float *scores;  // [sum q]
  int32_t n_rows;
};

struct TopkArgs {
  const float *scores;
  const int32_t *cu;       // [n + 1] offsets of each sequence's scores
  const int32_t *k;        // [n]
  const int32_t *out_off;  // [n] offsets into out
  int32_t *out;
};

struct MergeArgs {
  const uint16_t *o_a;
  const float *lse_a;
  const uint16_t *o_b;
  const float *lse_b;
  const uint8_t *mode;
  uint16_t *o;
  float *lse;  // or null
  int64_t n_pairs;  // rows * query heads
};

// The fixed device scratch of segkv_decode_noalloc (decode.hip): its size.
constexpr size_t kStaticScratchBytes = size_t(8) << 20;

}  // namespace segkv
