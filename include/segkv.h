/*
 * segkv.h -- C ABI of the segmented paged KV attention library (libsegkv.so).
 *
 * What the library computes.  Every (layer, KV head) has a class fixed
 * offline: a global head attends to the full causal context, a local head
 * only to a sliding window of the most recent tokens ("Xiaohongshu
 * Open-Sources RedKnot" page, section "What Happened", item 1).  The KV cache
 * is kept in pages per (layer, sequence, KV head) and per segment, so each
 * head stores and reads only the tokens it needs, and every head runs the
 * same fused variable-length attention with no attention mask built (same
 * page, item 3; "RedKnot: Head-Aware KV Reuse and SegPagedAttention" page,
 * section "The Three Core Mechanisms in Detail", third mechanism).
 *
 * Visibility (the reading this library implements): key j is visible to the
 * query at absolute position p iff j <= p and, for a local head with window
 * W, p - W < j.  Queries are the last tokens of their sequence: query t of a
 * sequence with kv_len cached tokens and q_len queries sits at
 * kv_len - q_len + t.  Query head h uses KV head h / (num_q_heads /
 * num_kv_heads).  Q and K are taken after any position encoding; a segment
 * whose keys were encoded at shifted positions takes a query rotation set
 * by segkv_set_relocation.
 *
 * Outputs: o = softmax(scale * q k^T restricted to visible keys) v, rounded
 * once to bf16, and lse = ln(sum over visible keys of exp(scale * q.k)) in
 * fp32.
 *
 * Memory.  Every device pointer is owned by the caller and must stay valid
 * until the work enqueued on the context's stream has completed.  Calls are
 * asynchronous on that stream; outputs are valid after the stream is
 * synchronised.  The context owns its host allocator state and its small
 * device tables.  A context is not thread-safe; use one per stream.
 *
 * Errors.  Every call validates its arguments and plans its allocation on the
 * host before anything is enqueued; a call that fails changes no state
 * (all-or-nothing).  segkv_last_error() returns a message for the last
 * failure.  After SEGKV_E_DEVICE the context must be destroyed.
 */
#ifndef SEGKV_H
#define SEGKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum segkv_status {
  SEGKV_OK = 0,
  SEGKV_E_INVAL = -1,  /* bad argument or shape */
  SEGKV_E_NOMEM = -2,  /* page pool or a fixed capacity exhausted */
  SEGKV_E_RANGE = -3,  /* unknown layer or sequence id */
  SEGKV_E_DEVICE = -4, /* HIP runtime error; destroy the context */
  SEGKV_E_STATE = -5   /* call not valid in this context or sequence state */
};

/* Kernel identifiers for segkv_read_timing(). */
enum segkv_kernel {
  SEGKV_KERNEL_SCATTER = 0,       /* KV append: writes new rows into pages   */
  SEGKV_KERNEL_PREFILL = 1,       /* varlen prefill attention                */
  SEGKV_KERNEL_DECODE_SPLIT = 2,  /* split-KV decode, partial (o, lse)      */
  SEGKV_KERNEL_COMBINE = 3,       /* log-sum-exp combine of split partials   */
  SEGKV_KERNEL_MERGE = 4,         /* head-decomposition merge (segkv_merge)  */
  SEGKV_KERNEL_SCORE = 5,         /* attention-mass token scores, MFMA pass  */
  SEGKV_KERNEL_SCORE_REDUCE = 6,  /* their fixed-order reduction              */
  SEGKV_KERNEL_TOPK = 7,          /* per-sequence top-k selection             */
  SEGKV_KERNEL_UPLOAD = 8,        /* copy of a call's tables to the device    */
  SEGKV_KERNEL_COUNT = 9
};

typedef struct segkv_ctx segkv_ctx;

typedef struct segkv_config {
  int32_t num_layers;
  int32_t num_q_heads;
  int32_t num_kv_heads;   /* num_q_heads % num_kv_heads == 0 */
  int32_t head_dim;       /* 64 or 128 */
  int32_t page_size;      /* tokens per page: 16, 32 or 64 */
  int32_t max_seqs;       /* sequence ids are 0 .. max_seqs-1 */
  int64_t num_pages;      /* pool capacity in pages, shared by every layer, sequence and KV head (< 2^31) */
  const int32_t *head_window; /* host [num_layers][num_kv_heads]: 0 = global, W >= 1 = local window of W tokens.
                                 Copied at create. */
  float softmax_scale;    /* 0 => 1/sqrt(head_dim) */
  uint64_t page_order_seed; /* 0 => free list hands out pages in index order; else a seeded permutation */
  void *k_pool;           /* device bf16, num_pages * page_size * head_dim elements: one page = page_size K rows
                             of one (layer, sequence, KV head).  Inside a page the rows go in pairs, and each
                             128-byte line holds the same 64-byte group of both rows of a pair. */
  void *v_pool;           /* device bf16, the same size: each V page is stored transposed (head_dim channel rows
                             of page_size keys), channel rows paired the same way when longer than 64 bytes.
                             The library alone reads and writes both pools. */
  void *stream;           /* hipStream_t for all device work; NULL = the default stream */
  /* Rotary position code of the queries, used only by segkv_set_relocation
     (zero-initialised fields give the defaults). */
  float rope_theta;       /* base of the rotary frequencies; 0 => 10000 */
  int32_t rope_style;     /* 0: rotate-half (channel i pairs with i + rope_dims/2);
                             1: interleaved (channels 2i and 2i+1 pair) */
  int32_t rope_dims;      /* rotary channels, the trailing ones of a head; 0 => head_dim; otherwise a
                             multiple of 16 in [16, head_dim].  Leading channels carry no position code. */
  /* Device scratch of every call: its tables (sequence and segment
     descriptors, page ids, work lists) and the split partials (o, lse) that
     the combine merges.  Owned by the caller, 256-byte aligned, at least
     segkv_workspace_bytes() bytes for the batches the caller will run.  NULL
     (device contexts): segkv_create allocates workspace_bytes bytes, or
     segkv_workspace_bytes(cfg, max_batch_q_tokens) when workspace_bytes is 0,
     and frees them in segkv_destroy.  No call allocates device memory after
     create.  Ignored by planning-only contexts. */
  void *workspace;
  uint64_t workspace_bytes;
  int32_t max_batch_q_tokens; /* largest query-token count of one prefill or token-score batch that the
                                 context's own workspace and host staging are sized for; 0 => 16384 */
  int32_t pad0;
} segkv_config;

/*
 * Device workspace that suffices for every call on batches of at most
 * max_seqs sequences and max_batch_q_tokens query tokens (prefill and token
 * scores; a decode batch is at most max_seqs sequences), when the segments
 * listed in one call hold at most num_pages page ids together (always true
 * without forks; sequences that share pages through segkv_fork list each
 * shared page once per sequence, so a batch of forks may need more) and the
 * prefill split knob is automatic.  The bound covers the prefill's split
 * partials (at most two per resident workgroup), the decode's stream-K
 * partials (one per segment piece) and the token scores' partial rows (one
 * per visible (query tile, key tile) pair, which grows with the square of a
 * global head's chunk).  A call that needs more than the workspace holds
 * fails with SEGKV_E_NOMEM before it enqueues anything or changes any
 * state.  Returns 0 for an invalid configuration or a negative token count.
 */
size_t segkv_workspace_bytes(const segkv_config *cfg, int32_t max_batch_q_tokens);

/*
 * Create a context: the head-class table (one window per (layer, KV head),
 * 0 = global: "Xiaohongshu Open-Sources RedKnot" page, "What Happened",
 * item 1, where each (layer, head) is classified offline as global or as
 * local with a sliding window) and the page pool of the per-(layer, head)
 * segmented storage (same page, item 3; "RedKnot: Head-Aware KV Reuse and
 * SegPagedAttention" page, "The Three Core Mechanisms in Detail", third
 * mechanism).  k_pool and v_pool both NULL gives a planning-only
 * context: it keeps the page allocator and tables on the host and makes no
 * HIP call at all (appends take k_new = v_new = NULL; prefill and decode
 * return SEGKV_E_STATE).  Returns SEGKV_OK and *out, or an error with *out =
 * NULL (message: segkv_last_error(NULL)).
 */
int segkv_create(const segkv_config *cfg, segkv_ctx **out);

/* Destroy a context (waits for its stream).  NULL is a no-op. */
void segkv_destroy(segkv_ctx *ctx);

/*
 * Append new KV rows to n_seqs sequences of one layer and allocate their
 * pages: each head's segment holds only the tokens that head needs
 * ("Xiaohongshu Open-Sources RedKnot" page, "What Happened", item 3), and
 * the kept blocks are paged without further copies ("RedKnot's Long-Context
 * Speedup Matters for AI Workflows" page, "Head-level split changes cache
 * behavior").
 *   seq_ids  host int32 [n_seqs], distinct, each in [0, max_seqs)
 *   cu_new   host int32 [n_seqs + 1], prefix sums of the new-token counts
 *   n_query  host int32 [n_seqs]: the last n_query[b] appended tokens of
 *            sequence b are the queries of the next prefill/decode call
 *            (0 <= n_query[b] <= new count; 0 = cache fill, no queries).
 *   k_new, v_new  device bf16 [cu_new[n_seqs]][num_kv_heads][head_dim]
 * For each KV head the segment keeps the tokens a pending or later query
 * can see: all tokens for a global head; for a local head of window W the
 * tokens from max(0, p_q - W + 1) rounded down to a page, where p_q =
 * kv_len - n_query is the earliest pending query.  Pages wholly below that
 * start return to the pool and new tokens below it are never stored.  The
 * segment start never moves back.  Fails with SEGKV_E_NOMEM (no change) if
 * the pool cannot hold the whole batch.  When new tokens land in a
 * partially filled page that a fork also holds (segkv_fork), the sequence
 * first gets a private copy of that page (copy-on-write, one extra page).
 * When the queries form a prefill chunk (more queries than sequences), the
 * append also builds the device tables of the prefill of exactly these
 * queries and its scatter launch copies them to the device; a following
 * segkv_prefill whose tables come out the same byte for byte, with no
 * other call in between that writes tables, uses them instead of
 * uploading its own.  Results are the same either way.
 */
int segkv_append_pages(segkv_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                       const int32_t *cu_new, const int32_t *n_query, const void *k_new,
                       const void *v_new);

/*
 * Varlen prefill attention of n_seqs sequences of one layer: the fused
 * variable-length attention over the per-head segment pages, global heads
 * over the full causal context and local heads over their window only
 * ("Xiaohongshu Open-Sources RedKnot" page, "What Happened", items 1 and 3).
 * Result: o = softmax(scale q k^T) v per (query, query head) over the keys
 * that head sees, lse = ln of that softmax's denominator (natural log, with
 * the scale applied).
 *   seq_ids  host int32 [n_seqs]
 *   cu_q     host int32 [n_seqs + 1], prefix sums of q_len; q_len may be 0;
 *            each q_len must not reach before that sequence's earliest
 *            pending query (kv_len - q_len >= p_q).
 *   q        device bf16 [cu_q[n_seqs]][num_q_heads][head_dim]
 *   o        device bf16 [cu_q[n_seqs]][num_q_heads][head_dim]
 *   lse      device fp32 [cu_q[n_seqs]][num_q_heads], or NULL
 */
int segkv_prefill(segkv_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                  const int32_t *cu_q, const void *q, void *o, float *lse);

/*
 * One-token decode of n_seqs sequences of one layer (the query is the last
 * cached token of each sequence): the same attention as segkv_prefill for
 * one query row ("Xiaohongshu Open-Sources RedKnot" page, "What Happened",
 * items 1 and 3).  The pages give no decode kernel; the split over
 * workgroups and the combine below are this library's design.  The visible pages of all (sequence, KV
 * head) segments are split evenly over the GPU's workgroups (a segment may
 * be split across several); partial results are merged with a log-sum-exp
 * combine.  A work item takes up to 16 query heads of a KV group; a group of
 * more (num_q_heads / num_kv_heads > 16) is taken as blocks of 16, each of
 * which reads the segment's visible pages.
 *   q, o     device bf16 [n_seqs][num_q_heads][head_dim]
 *   lse      device fp32 [n_seqs][num_q_heads], or NULL
 */
int segkv_decode(segkv_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                 const void *q, void *o, float *lse);

/*
 * segkv_decode for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels and results, but the call's tables and split partials go to
 * a fixed device scratch array of 8 MiB that the library holds on each GPU
 * for the life of the process, instead of the context's workspace.  The
 * call allocates nothing (no device, pinned or host buffer, no timing
 * event: kernel timing is not recorded for it).  A batch whose tables and
 * partials exceed 8 MiB, or whose tables exceed the host staging buffers
 * sized at create, fails with SEGKV_E_NOMEM before anything is enqueued.
 * Every context on a GPU shares that GPU's array and each call overwrites
 * it: calls that overlap in time on one GPU (two streams, two contexts,
 * two threads) race and must not be issued.  Arguments and errors are
 * those of segkv_decode.
 */
int segkv_decode_noalloc(segkv_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                         const void *q, void *o, float *lse);

/*
 * Query-side RoPE relocation ("RedKnot-MLA: Multi-Head Offline-Online Reuse
 * for DeepSeek-V4 Long-Context Serving" review, "Summary"; the paper page's
 * abstract).  A reused document's KV is encoded at canonical positions
 * (the document starting at 0); placed at offset delta in a live request,
 * its keys keep that encoding and the queries are turned back by delta
 * instead.  A rotary code makes q.k depend only on the position difference,
 * so the scores equal those of keys re-encoded at their true positions.
 *
 * Sets the offset of every (layer, KV head) segment of one sequence:
 *   deltas  host int32 [num_layers][num_kv_heads], or NULL for all zero.
 * Later prefill and decode calls rotate each query of KV head g's group by
 * -delta (pair i of the rotary block by angle -delta * rope_theta^(-2i /
 * rope_dims)) in fp32 from an fp64 cos/sin table, and round the result once
 * to bf16 before scoring.  delta = 0 leaves the queries untouched.  Offsets
 * persist until changed or until segkv_release, which clears them.  Valid in
 * a planning-only context (host state only).
 */
int segkv_set_relocation(segkv_ctx *ctx, int32_t seq_id, const int32_t *deltas);

/*
 * Head-decomposition merge ("RedKnot: Head-Aware KV Reuse and
 * SegPagedAttention" page, "The Three Core Mechanisms in Detail", first
 * mechanism; "RedKnot-MLA: Multi-Head Offline-Online Reuse for DeepSeek-V4
 * Long-Context Serving" review, "Key claims under review" and
 * "Strengths").  Local-head results prepared offline (partial A) are
 * combined with results computed online (partial B): Global heads,
 * protected rows, and the keys a reused document's rows see outside the
 * document.  Each (row, query head) pair takes, by its mode byte:
 *   SEGKV_MERGE_TAKE_A  o = o_a, lse = lse_a (bit for bit)
 *   SEGKV_MERGE_TAKE_B  o = o_b, lse = lse_b (bit for bit)
 *   SEGKV_MERGE_LSE     the softmax over the union of the two parts' key
 *                       sets (they must be disjoint): lse = ln(e^lse_a +
 *                       e^lse_b), o = e^(lse_a - lse) o_a + e^(lse_b - lse)
 *                       o_b, evaluated in fp32 and rounded once to bf16.  A
 *                       part with lse = -inf weighs 0; if both are -inf then
 *                       o = 0, lse = -inf.  Any mode value >= 2 merges.
 * Only the parts a pair's mode needs are read.
 *   o_a, o_b      device bf16 [n_rows][num_q_heads][head_dim], 16-byte aligned
 *   lse_a, lse_b  device fp32 [n_rows][num_q_heads] (natural log)
 *   mode          device uint8 [n_rows][num_q_heads]
 *   o             device bf16 [n_rows][num_q_heads][head_dim], 16-byte aligned;
 *                 may be o_a or o_b (in place)
 *   lse           device fp32 [n_rows][num_q_heads] or NULL; may be lse_a or lse_b
 * Other overlaps between inputs and outputs are not allowed.  Device
 * contexts only (SEGKV_E_STATE in a planning context).
 */
enum segkv_merge_mode {
  SEGKV_MERGE_TAKE_A = 0,
  SEGKV_MERGE_TAKE_B = 1,
  SEGKV_MERGE_LSE = 2
};
int segkv_merge(segkv_ctx *ctx, int64_t n_rows, const void *o_a, const float *lse_a, const void *o_b,
                const float *lse_b, const uint8_t *mode, void *o, float *lse);

/*
 * Fork ("RedKnot: Head-Aware KV Reuse and SegPagedAttention" page, sections
 * "Getting Started: Repository Layout and Entry Points" and "Experimental
 * Features and Current Limitations": request forks with copy-on-write
 * append).  dst_seq, which must hold no tokens in any layer, becomes a
 * copy of src_seq: same lengths, pending queries and relocation offsets,
 * and the same physical pages in every (layer, KV head) segment, shared by
 * reference count.  No page is allocated and no device work is enqueued.
 * Full shared pages are never written again; an append that writes into a
 * shared partially filled tail page copies it first (segkv_append_pages).
 * A page returns to the pool when its last holder releases or trims it.
 * Errors: SEGKV_E_RANGE for ids out of range, SEGKV_E_INVAL if src == dst,
 * SEGKV_E_STATE if dst is not empty.  Valid in a planning-only context.
 */
int segkv_fork(segkv_ctx *ctx, int32_t src_seq, int32_t dst_seq);

/*
 * Attention-mass token scores, the router of the sparse FFN ("Xiaohongshu
 * Open-Sources RedKnot" page, "What Happened" item 2 and "Why Sparse FFN
 * Matters for Agent Workloads"; "RedKnot: Head-Aware KV Reuse and
 * SegPagedAttention" page, "The Three Core Mechanisms in Detail", second
 * mechanism: dense FFN only on the top-k tokens by attention score).
 * A second pass after segkv_prefill with the same seq_ids, cu_q and q (and
 * its lse): for each sequence b and each token j of its query chunk (as a
 * key),
 *   scores[cu_q[b] + (j - (kv_len - q_len))] = sum over the chunk's query
 *   rows t and all query heads h that see j of exp(scale q_{t,h}.k_j -
 *   lse_{t,h}),
 * the attention mass j receives (fp32; each probability row sums to 1, so a
 * sequence's scores add up to at most q_len * num_q_heads).  Relocation
 * offsets apply as in the prefill.  The sum is taken in a fixed order:
 * results are bitwise reproducible and do not depend on tuning knobs.
 *   q      device bf16 [cu_q[n_seqs]][num_q_heads][head_dim]
 *   lse    device fp32 [cu_q[n_seqs]][num_q_heads], from segkv_prefill
 *   scores device fp32 [cu_q[n_seqs]]
 * Same argument checks as segkv_prefill; seq_ids must be distinct.
 */
int segkv_token_scores(segkv_ctx *ctx, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                       const int32_t *cu_q, const void *q, const float *lse, float *scores);

/*
 * Top-k tokens of each sequence by score (for example segkv_token_scores'
 * output): the k[b] highest of scores[cu_n[b] .. cu_n[b+1]), ties broken
 * towards the lower index, written as indices local to the sequence (0 ..
 * n_b - 1) in ascending order to out_idx[sum_{b'<b} k[b'] ..].  Scores must
 * be >= 0 (they are ordered by their bit patterns).
 *   cu_n    host int32 [n_seqs + 1], prefix sums of the per-sequence counts
 *   scores  device fp32 [cu_n[n_seqs]]
 *   k       host int32 [n_seqs], 0 <= k[b] <= n_b
 *   out_idx device int32 [sum k]
 */
int segkv_topk(segkv_ctx *ctx, int32_t n_seqs, const int32_t *cu_n, const float *scores, const int32_t *k,
               int32_t *out_idx);

/* Drop every page reference of a sequence (all layers, all heads): pages no
 * other sequence holds return to the pool.  Resets its length to 0 and
 * clears its relocation offsets. */
int segkv_release(segkv_ctx *ctx, int32_t seq_id);

/*
 * Introspection of one segment.  Writes the logical index of the first token
 * the segment holds, the sequence length and the page count; copies up to
 * cap physical page ids (page i holds tokens first_token + i*page_size ...)
 * into page_ids when it is not NULL.
 */
int segkv_page_table(const segkv_ctx *ctx, int32_t layer, int32_t seq_id, int32_t kv_head,
                     int32_t *first_token, int32_t *kv_len, int32_t *n_pages, int32_t *page_ids,
                     int32_t cap);

/* Pages currently on the free list, or a negative status. */
int64_t segkv_free_pages(const segkv_ctx *ctx);

/*
 * Kernel timing with HIP events recorded on the context's stream around each
 * launch of the kernels selected by kernel_mask (bit k = enum segkv_kernel
 * k; SEGKV_TIME_ALL selects all; 0 switches timing off).  Setting the mask
 * clears the counters.  segkv_read_timing synchronises the recorded events
 * and returns the summed duration (ms) and launch count of one kernel.
 */
#define SEGKV_TIME_ALL ((1 << SEGKV_KERNEL_COUNT) - 1)
int segkv_set_timing(segkv_ctx *ctx, int32_t kernel_mask);
int segkv_read_timing(segkv_ctx *ctx, int32_t kernel, double *total_ms, int64_t *launches);

/*
 * Tuning knobs (values <= 0 restore the default):
 *   SEGKV_TUNE_DECODE_MIN_PAGES        decode cuts the batch's visible pages
 *                                      into equal shares, one per workgroup,
 *                                      using the GPU's resident workgroup
 *                                      slots but no share below this many
 *                                      pages (default 8)
 *   SEGKV_TUNE_PREFILL_SPLIT_TILES     a prefill work item covering more
 *                                      64-key tiles than this is split across
 *                                      workgroups and merged by the combine
 *                                      kernel.  Default: automatic, the
 *                                      batch's total tiles over the GPU's
 *                                      resident workgroup slots (at least
 *                                      16); a huge value disables splitting.
 *                                      The token-score pass cuts its items
 *                                      into pieces of at most this many tiles
 *                                      too (automatic: the total over twice
 *                                      its resident workgroups, at least 16).
 *   SEGKV_TUNE_PREFILL_ORDER           0 (default): the work list is taken
 *                                      longest first; 1: the list is cut into
 *                                      eight cost-balanced runs grouped by
 *                                      head, each sorted longest first, and
 *                                      the runs are interleaved.
 *   SEGKV_TUNE_PREFILL_KERNEL          0 (default) or 1: the prefill kernel of
 *                                      8 waves x 32 rows (two waves per SIMD);
 *                                      2: the kernel of 4 waves x 64 rows (one
 *                                      wave per SIMD, each K/V^T operand read
 *                                      from LDS feeds two products, softmax
 *                                      pipelined under the products);
 *                                      3: the 8 x 32-row kernel as two groups
 *                                      of four waves one phase apart (one
 *                                      group's products beside the other's
 *                                      softmax), over per-workgroup item lists
 *                                      balanced on the host;
 *                                      4: the 8 x 32-row kernel software
 *                                      pipelined across tiles (each tile's
 *                                      exponentials under the next tile's QK
 *                                      products, its mask and max under the
 *                                      PV products);
 *                                      5: two workgroups per CU, each of 4
 *                                      waves x 32 rows over 128-row work
 *                                      items with two K/V stages (needs
 *                                      num_q_heads / num_kv_heads <= 128).
 *                                      Values outside 0 .. 5 are rejected
 *                                      (SEGKV_E_INVAL).
 * Results do not depend on the knobs beyond fp32 rounding of split merges.
 */
enum segkv_tune {
  SEGKV_TUNE_DECODE_MIN_PAGES = 0,
  SEGKV_TUNE_PREFILL_SPLIT_TILES = 1,
  SEGKV_TUNE_PREFILL_ORDER = 2,
  SEGKV_TUNE_PREFILL_KERNEL = 3
};
int segkv_set_tuning(segkv_ctx *ctx, int32_t knob, int64_t value);

/* Message for the last failure on ctx (ctx = NULL: the last failed create). */
const char *segkv_last_error(const segkv_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* SEGKV_H */
