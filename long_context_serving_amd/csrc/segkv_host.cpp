// Host side of libsegkv: the C ABI, the per-head segment page allocator and
// the per-call device table builder.  Device work is in the csrc/*.hip kernels.
//
// The allocator follows the storage rule of SegPagedAttention: KV pages are
// kept per (layer, head) and per segment, and a head stores only the tokens
// it needs ("Xiaohongshu Open-Sources RedKnot" page, section "What
// Happened", item 3; "RedKnot: Head-Aware KV Reuse and SegPagedAttention"
// page, section "The Three Core Mechanisms in Detail", third mechanism).  A
// local head keeps the pages that a pending or later query can still see;
// everything below its window returns to the pool and is never written.

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <limits>
#include <random>
#include <string>
#include <vector>

#include "segkv.h"
#include "segkv_internal.h"
#include "segkv_launch.h"
#include "segkv_sched.h"

using namespace segkv;

segkv::LaunchEvents &segkv::launch_events() {
  static thread_local LaunchEvents ev;
  return ev;
}

namespace {

thread_local std::string g_create_error;

constexpr int kStages = 32;     // pinned staging slots, used in ring order
constexpr int kStageGroup = 8;  // slots covered by one completion event
constexpr int kDefaultDecodeMinPages = 8;
// Cost of one decode piece (its query load and partial merge) in keys of
// streaming, from per-workgroup timings: about one 64-key chunk.
constexpr int64_t kDecodePieceCostKeys = 64;
constexpr size_t kPrestageRoom = 64 << 10;  // initial room for prefill tables staged by an append
constexpr int kDefaultPrefillSplitTiles = 0;  // automatic
constexpr int64_t kMinSplitTiles = 16;
// Cost of starting an item and writing its output, in tile steps, when the
// two-group prefill's items are balanced over its workgroups.
constexpr int64_t kItemCostTiles = 2;
// SEGKV_TUNE_PREFILL_KERNEL values of the two variants beside the default kernel
constexpr int32_t kPrefillWide = 2;
constexpr int32_t kPrefillTwoGroup = 3;
constexpr int32_t kPrefillPipelined = 4;
constexpr int32_t kPrefillDuo = 5;

struct Segment {
  int32_t first_token = 0;
  int32_t delta = 0;           // query relocation offset (0 = none)
  std::vector<int32_t> pages;  // live pages are pages[head, size)
  size_t head = 0;
  int32_t n_live() const { return static_cast<int32_t>(pages.size() - head); }
  const int32_t *live() const { return pages.data() + head; }
  void drop_front(int32_t n) {
    head += static_cast<size_t>(n);
    if (head == pages.size()) {
      pages.clear();
      head = 0;
    } else if (head >= 256 && head * 2 >= pages.size()) {
      pages.erase(pages.begin(), pages.begin() + static_cast<std::ptrdiff_t>(head));
      head = 0;
    }
  }
};

struct SeqLayer {
  int32_t kv_len = 0;
  int32_t pending_from = 0;  // earliest query position a later call may use
};

struct TimedLaunch {
  int kernel;
  hipEvent_t start;
  hipEvent_t stop;
};

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace

struct segkv_ctx {
  // configuration
  int32_t L = 0, Hq = 0, Hkv = 0, D = 0, P = 0, S = 0, G = 0;
  int64_t num_pages = 0;
  float scale = 0.f;
  std::vector<int32_t> window;  // [L][Hkv]
  double rope_theta = 10000.0;
  int32_t rope_style = 0;  // 0 rotate-half, 1 interleaved
  int32_t rope_dims = 0;   // trailing rotary channels
  uint16_t *k_pool = nullptr;
  uint16_t *v_pool = nullptr;
  hipStream_t stream = nullptr;
  bool planning = false;

  // allocator state
  std::vector<int32_t> free_list;  // stack; back() is handed out first
  std::vector<int32_t> refcnt;     // [num_pages]: segments holding each page (0 = free)
  std::vector<Segment> segs;       // [L][S][Hkv]
  std::vector<SeqLayer> seq_layer; // [L][S]

  // Device workspace: each call puts its tables at the start and its split
  // partials after them (at a 256-byte boundary).  Caller-owned unless the
  // config left it NULL.
  char *ws = nullptr;
  size_t ws_bytes = 0;
  bool ws_owned = false;
  int32_t max_q = 0;  // query tokens the staging was sized for
  char *fixed_scratch = nullptr;  // this device's copy of the fixed scratch (segkv_decode_noalloc)
  // host staging
  char *h_stage[kStages] = {};
  char *h_stage_dev[kStages] = {};  // the same pinned memory as seen by kernels
  size_t h_stage_cap[kStages] = {};
  hipEvent_t stage_ev[kStages / kStageGroup] = {};  // recorded when the ring leaves the group
  bool stage_used[kStages / kStageGroup] = {};
  int stage_next = 0;
  // Prefill tables put on the device by an append's scatter launch: valid
  // while nothing else has written the workspace's tables since (pre_buf =
  // their bytes).
  std::vector<char> pre_buf, plan_buf;
  bool pre_valid = false;
  size_t pre_room = kPrestageRoom;  // staging room an append keeps for them
  int32_t num_cus = 0;

  // tuning
  int32_t decode_pps = kDefaultDecodeMinPages;  // minimum pages per decode workgroup
  int64_t prefill_split_tiles = kDefaultPrefillSplitTiles;  // 0 = automatic
  int32_t prefill_order = 0;  // 0 = longest-first, 1 = XCD-aware
  int32_t prefill_kernel = 0;  // 0/1 = 8 waves x 32 rows in step (default), 2 = 4 waves x 64 rows, 3 = two-group
                               // schedule, 4 = pipelined, 5 = two workgroups per CU of 4 waves x 32 rows

  // timing
  int32_t timing_mask = 0;  // bit k: record events around kernel k
  std::vector<TimedLaunch> pending;
  std::vector<hipEvent_t> event_pool;
  double tot_ms[SEGKV_KERNEL_COUNT] = {};
  int64_t launches[SEGKV_KERNEL_COUNT] = {};

  // scratch reused across calls
  std::vector<int32_t> scratch_i32;
  std::vector<int32_t> scratch_wg;     // per-workgroup item offsets of the two-group prefill
  std::vector<int32_t> scratch_owner;  // workgroup of each prefill item
  std::vector<int32_t> scratch_order;  // prefill items grouped by workgroup
  std::vector<int64_t> scratch_cost;
  std::vector<int32_t> scratch_cnt;  // counting sort of the prefill work list (an append plans a prefill too)
  std::vector<int32_t> scratch_deltas;  // distinct nonzero offsets of the current call
  std::vector<int32_t> scratch_release;  // pages whose reference an append drops after it allocated
  std::vector<PrefillItem> scratch_pitems;
  std::vector<CombineItem> scratch_citems;

  std::string err;

  Segment &seg(int32_t layer, int32_t s, int32_t g) {
    return segs[(static_cast<size_t>(layer) * S + s) * Hkv + g];
  }
  const Segment &seg(int32_t layer, int32_t s, int32_t g) const {
    return segs[(static_cast<size_t>(layer) * S + s) * Hkv + g];
  }
  SeqLayer &sl(int32_t layer, int32_t s) { return seq_layer[static_cast<size_t>(layer) * S + s]; }
  const SeqLayer &sl(int32_t layer, int32_t s) const {
    return seq_layer[static_cast<size_t>(layer) * S + s];
  }
  int32_t win(int32_t layer, int32_t g) const { return window[static_cast<size_t>(layer) * Hkv + g]; }

  // Pages are shared between forked sequences; a page returns to the free
  // list when its last holder drops it.
  int32_t take_page() {
    // The caller has checked that the batch fits; an empty list here is a
    // bug in that check, never a state to continue from.
    if (free_list.empty()) {
      std::fprintf(stderr, "segkv: internal error: page allocation from an empty free list\n");
      std::abort();
    }
    const int32_t id = free_list.back();
    free_list.pop_back();
    refcnt[static_cast<size_t>(id)] = 1;
    return id;
  }
  void drop_page(int32_t id) {
    if (--refcnt[static_cast<size_t>(id)] == 0) free_list.push_back(id);
  }

  int fail(int code, const char *fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    err = buf;
    return code;
  }
  int device_fail(hipError_t e, const char *what) {
    return fail(SEGKV_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
  }
};

namespace {

// Segment start rule for a local head: keep keys a pending or later query
// can see, i.e. from max(0, p_q - W + 1), rounded down to a page.
int32_t local_segment_start(int32_t kv_len, int32_t n_query, int32_t window, int32_t page) {
  int64_t p_q = static_cast<int64_t>(kv_len) - n_query;
  int64_t lo = std::max<int64_t>(0, p_q - window + 1);
  return static_cast<int32_t>(page * (lo / page));
}

// ---- staging / upload --------------------------------------------------

// Pinned staging buffer `slot` holds at least `bytes` (the caller has made
// sure no enqueued work still reads it).  Slots are sized at create for the
// largest tables of the context's batch range; only a larger call (a huge
// cache-fill append, a token-score call past that range) grows one.
int ensure_stage(segkv_ctx *c, int slot, size_t bytes) {
  if (c->h_stage_cap[slot] >= bytes) return SEGKV_OK;
  if (c->h_stage[slot]) {
    hipError_t e = hipHostFree(c->h_stage[slot]);
    if (e != hipSuccess) return c->device_fail(e, "hipHostFree");
    c->h_stage[slot] = nullptr;
    c->h_stage_cap[slot] = 0;
  }
  size_t cap = std::max<size_t>(align_up(bytes, 1 << 16), 1 << 16);
  hipError_t e = hipHostMalloc(reinterpret_cast<void **>(&c->h_stage[slot]), cap, hipHostMallocDefault);
  if (e != hipSuccess) return c->device_fail(e, "hipHostMalloc(stage)");
  e = hipHostGetDevicePointer(reinterpret_cast<void **>(&c->h_stage_dev[slot]), c->h_stage[slot], 0);
  if (e != hipSuccess) return c->device_fail(e, "hipHostGetDevicePointer(stage)");
  c->h_stage_cap[slot] = cap;
  return SEGKV_OK;
}

// Every call that stages tables takes the next pinned buffer of a ring of
// kStages; its kernels read the buffer in place or through the upload
// kernel.  One completion event covers a group of kStageGroup buffers, so
// most calls record no event: an event marker between two kernels on the
// stream lengthens the gap between them.
int acquire_stage(segkv_ctx *c, size_t bytes, char **out, int *slot_out) {
  int slot = c->stage_next;
  c->stage_next = (c->stage_next + 1) % kStages;
  if (slot % kStageGroup == 0) {
    // Entering group g: the work enqueued so far is all the work that reads
    // the previous group's slots, so one event marks them free.  Group g
    // itself is reused once the event recorded when the ring left it fires.
    constexpr int n_groups = kStages / kStageGroup;
    const int g = slot / kStageGroup;
    const int prev = (g + n_groups - 1) % n_groups;
    hipError_t e = hipEventRecord(c->stage_ev[prev], c->stream);
    if (e != hipSuccess) return c->device_fail(e, "hipEventRecord(stage)");
    c->stage_used[prev] = true;
    if (c->stage_used[g]) {
      e = hipEventSynchronize(c->stage_ev[g]);
      if (e != hipSuccess) return c->device_fail(e, "hipEventSynchronize(stage)");
    }
  }
  const int rc = ensure_stage(c, slot, bytes);
  if (rc) return rc;
  *out = c->h_stage[slot];
  *slot_out = slot;
  return SEGKV_OK;
}

// Where a call's tables and partials go: tables at base, partials at the
// next 256-byte boundary.  Fails (before anything is enqueued) when they do
// not fit in cap bytes.
int carve(segkv_ctx *c, char *base, size_t cap, size_t table_bytes, size_t part_bytes, float **parts) {
  const size_t off = align_up(table_bytes, 256);
  if (off + part_bytes > cap)
    return c->fail(SEGKV_E_NOMEM,
                   "workspace too small: this call needs %zu bytes of tables and %zu of partials, the workspace "
                   "holds %zu (size it with segkv_workspace_bytes)",
                   table_bytes, part_bytes, cap);
  *parts = part_bytes ? reinterpret_cast<float *>(base + off) : nullptr;
  return SEGKV_OK;
}

int timed_begin(segkv_ctx *c, TimedLaunch *t, int kernel);
int timed_end(segkv_ctx *c, TimedLaunch *t);

// Tables go to device memory through a small copy kernel on the context's
// stream (it reads the pinned staging buffer directly): a DMA-engine copy
// between kernels costs a queue hand-off that is several times the copy.
int upload(segkv_ctx *c, int slot, size_t bytes, char *dst) {
  if (dst == c->ws) c->pre_valid = false;
  TimedLaunch t{};
  int rc = timed_begin(c, &t, SEGKV_KERNEL_UPLOAD);
  if (rc) return rc;
  hipError_t e = launch_upload(dst, c->h_stage_dev[slot], bytes, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "upload launch");
  return timed_end(c, &t);
}

// ---- timing --------------------------------------------------------------

// A timed launch: timed_begin takes two events from the pool and hands them
// to the next launch on this thread, whose dispatch stamps the kernel's own
// start and end; timed_end takes them back (a launcher that had nothing to
// launch leaves them unused, and they return to the pool).
int timed_begin(segkv_ctx *c, TimedLaunch *t, int kernel) {
  t->kernel = -1;
  launch_events() = LaunchEvents{};
  if (!(c->timing_mask & (1 << kernel))) return SEGKV_OK;
  t->kernel = kernel;
  for (hipEvent_t *ev : {&t->start, &t->stop}) {
    if (!c->event_pool.empty()) {
      *ev = c->event_pool.back();
      c->event_pool.pop_back();
    } else {
      hipError_t e = hipEventCreate(ev);
      if (e != hipSuccess) return c->device_fail(e, "hipEventCreate");
    }
  }
  launch_events() = LaunchEvents{t->start, t->stop, false};
  return SEGKV_OK;
}

int timed_end(segkv_ctx *c, TimedLaunch *t) {
  const bool used = launch_events().used;
  launch_events() = LaunchEvents{};
  if (t->kernel < 0) return SEGKV_OK;
  if (used) {
    c->pending.push_back(*t);
  } else {
    c->event_pool.push_back(t->start);
    c->event_pool.push_back(t->stop);
  }
  return SEGKV_OK;
}

int drain_timing(segkv_ctx *c) {
  for (const TimedLaunch &t : c->pending) {
    hipError_t e = hipEventSynchronize(t.stop);
    if (e != hipSuccess) return c->device_fail(e, "hipEventSynchronize(timing)");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, t.start, t.stop);
    if (e != hipSuccess) return c->device_fail(e, "hipEventElapsedTime");
    c->tot_ms[t.kernel] += ms;
    c->launches[t.kernel] += 1;
    c->event_pool.push_back(t.start);
    c->event_pool.push_back(t.stop);
  }
  c->pending.clear();
  return SEGKV_OK;
}

// ---- shared validation ---------------------------------------------------

int check_layer_seqs(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids) {
  if (layer < 0 || layer >= c->L) return c->fail(SEGKV_E_RANGE, "layer %d out of range [0, %d)", layer, c->L);
  if (n_seqs < 0) return c->fail(SEGKV_E_INVAL, "n_seqs < 0");
  if (n_seqs > c->S) return c->fail(SEGKV_E_INVAL, "n_seqs %d exceeds max_seqs %d", n_seqs, c->S);
  if (n_seqs > 0 && !seq_ids) return c->fail(SEGKV_E_INVAL, "seq_ids is NULL");
  for (int32_t b = 0; b < n_seqs; ++b)
    if (seq_ids[b] < 0 || seq_ids[b] >= c->S)
      return c->fail(SEGKV_E_RANGE, "seq id %d out of range [0, %d)", seq_ids[b], c->S);
  return SEGKV_OK;
}

// Byte offsets of the per-call sequence tables: SeqDesc, SegDesc, page ids
// and relocation tables, each 16-byte aligned.
struct SeqTables {
  size_t seg_off = 0, pid_off = 0, rope_off = 0, bytes = 0;
};

// Sizes the tables of a batch; collects the distinct nonzero relocation
// offsets of its segments into c->scratch_deltas (sorted).
SeqTables seq_tables_layout(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids) {
  int64_t pages = 0;
  std::vector<int32_t> &deltas = c->scratch_deltas;
  deltas.clear();
  for (int32_t b = 0; b < n_seqs; ++b)
    for (int32_t g = 0; g < c->Hkv; ++g) {
      const Segment &sg = c->seg(layer, seq_ids[b], g);
      pages += sg.n_live();
      if (sg.delta) deltas.push_back(sg.delta);
    }
  std::sort(deltas.begin(), deltas.end());
  deltas.erase(std::unique(deltas.begin(), deltas.end()), deltas.end());
  SeqTables t;
  t.seg_off = align_up(sizeof(SeqDesc) * n_seqs, 16);
  t.pid_off = t.seg_off + align_up(sizeof(SegDesc) * static_cast<size_t>(n_seqs) * c->Hkv, 16);
  t.rope_off = t.pid_off + align_up(sizeof(int32_t) * static_cast<size_t>(pages), 16);
  t.bytes = t.rope_off + sizeof(float) * 2 * static_cast<size_t>(c->D) * deltas.size();
  return t;
}

// Relocation table of one offset: channel ch of a query becomes cos[ch] *
// q[ch] + ssin[ch] * q[partner(ch)], the rotation of its pair by -delta
// radians times the pair's frequency rope_theta^(-2i / rope_dims).  The
// first element of a pair takes -sin, the second +sin.  Evaluated in fp64,
// stored in fp32.
void write_rope_table(const segkv_ctx *c, int32_t delta, float *cs) {
  const int32_t D = c->D, R = c->rope_dims, lo = D - R;
  for (int32_t ch = 0; ch < D; ++ch) {
    if (ch < lo) {
      cs[ch] = 1.f;
      cs[D + ch] = 0.f;
      continue;
    }
    const int32_t j = ch - lo;
    const int32_t pair = c->rope_style == 0 ? j % (R / 2) : j / 2;
    const bool first = c->rope_style == 0 ? j < R / 2 : (j % 2) == 0;
    const double ang = -static_cast<double>(delta) * std::pow(c->rope_theta, -2.0 * pair / R);
    cs[ch] = static_cast<float>(std::cos(ang));
    cs[D + ch] = static_cast<float>(first ? -std::sin(ang) : std::sin(ang));
  }
}

void write_seq_tables(const segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids,
                      const int32_t *q_start, const int32_t *q_len, const SeqTables &t, char *dst) {
  SeqDesc *sd = reinterpret_cast<SeqDesc *>(dst);
  SegDesc *gd = reinterpret_cast<SegDesc *>(dst + t.seg_off);
  int32_t *pid = reinterpret_cast<int32_t *>(dst + t.pid_off);
  float *rope = reinterpret_cast<float *>(dst + t.rope_off);
  const std::vector<int32_t> &deltas = c->scratch_deltas;
  for (size_t i = 0; i < deltas.size(); ++i) write_rope_table(c, deltas[i], rope + i * 2 * c->D);
  int32_t off = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const SeqLayer &s = c->sl(layer, seq_ids[b]);
    sd[b] = SeqDesc{s.kv_len, q_start ? q_start[b] : b, q_len ? q_len[b] : 1, 0};
    for (int32_t g = 0; g < c->Hkv; ++g) {
      const Segment &sg = c->seg(layer, seq_ids[b], g);
      int32_t rope_off = -1;
      if (sg.delta) {
        const size_t i = static_cast<size_t>(std::lower_bound(deltas.begin(), deltas.end(), sg.delta) - deltas.begin());
        rope_off = static_cast<int32_t>(i * 2 * c->D);
      }
      gd[static_cast<size_t>(b) * c->Hkv + g] =
          SegDesc{sg.first_token, off, sg.n_live(), c->win(layer, g), rope_off, 0, 0, 0};
      std::memcpy(pid + off, sg.live(), sizeof(int32_t) * sg.n_live());
      off += sg.n_live();
    }
  }
}

// (query position, query head) rows of one prefill work item for the
// context's prefill kernel.
int32_t prefill_item_rows(const segkv_ctx *c) {
  return c->prefill_kernel == kPrefillDuo ? kPrefillDuoRows : kPrefillRows;
}

// A prefill call's device tables, in upload order: sequence tables, work
// items, combine items, the work-queue counter (16 bytes, zero), then the
// per-workgroup item ranges of the two-group kernel.
struct PrefillPlan {
  SeqTables tl;
  size_t tbytes = 0, ibytes = 0, cbytes = 0, wbytes = 0, bytes = 0;
  int32_t n_items = 0, n_parts = 0, n_wgs = 0;
};

// Plans a prefill of the queries cu_q over the current state: the work list
// (c->scratch_pitems, c->scratch_citems) and the tables, written to out
// (resized to pp->bytes).  Bytes the tables do not set are zero, so two
// equal plans are equal byte for byte.
void build_prefill_plan(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const int32_t *cu_q,
                        PrefillPlan *pp, std::vector<char> *out) {
  // Work items: (seq, kv head, q tile) over the KV tiles the rows can see.
  const int32_t G = c->G;
  const int32_t rows = prefill_item_rows(c) / G;  // query positions per work item
  const int64_t wg_per_cu = c->prefill_kernel == kPrefillDuo ? kPrefillDuoWgPerCu : kPrefillWgPerCu;
  std::vector<PrefillItem> &items = c->scratch_pitems;
  std::vector<CombineItem> &citems = c->scratch_citems;
  items.clear();
  citems.clear();
  int64_t total_cost = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int32_t ql = cu_q[b + 1] - cu_q[b];
    const SeqLayer &s = c->sl(layer, seq_ids[b]);
    for (int32_t g = 0; g < c->Hkv; ++g) {
      const int32_t w = c->win(layer, g);
      // Last q tile first: for a global head the longest rows come first.
      for (int32_t qt = (ql + rows - 1) / rows - 1; qt >= 0; --qt) {
        const int32_t p_min = s.kv_len - ql + qt * rows;
        const int32_t p_max = s.kv_len - ql + std::min((qt + 1) * rows, ql) - 1;
        const int32_t lo = w > 0 ? std::max(0, p_min - w + 1) : 0;
        const int32_t tb = lo / kTileKeys;
        const int32_t te = p_max / kTileKeys + 1;
        items.push_back(PrefillItem{b, g, qt, tb, te, -1, 0, 0});
        total_cost += te - tb;
      }
    }
  }
  // Split rows that would outlast the average share of one workgroup slot;
  // their parts are merged by the combine kernel.
  int64_t split = c->prefill_split_tiles;
  if (split <= 0) {
    const int64_t slots = std::max<int64_t>(1, static_cast<int64_t>(c->num_cus) * wg_per_cu);
    split = std::max<int64_t>(kMinSplitTiles, ceil_div(total_cost, slots));
  }
  int32_t n_parts = 0;
  int64_t max_cost = 0;
  {
    std::vector<PrefillItem> expanded;
    expanded.reserve(items.size() + items.size() / 4);
    for (const PrefillItem &x : items) {
      const int64_t cost = x.tile_end - x.tile_begin;
      if (cost > split) {
        const int32_t ns = static_cast<int32_t>(ceil_div(cost, split));
        const int32_t per = static_cast<int32_t>(ceil_div(cost, ns));
        const int32_t part0 = n_parts;
        int32_t k = 0;
        for (int32_t t0 = x.tile_begin; t0 < x.tile_end; t0 += per, ++k)
          expanded.push_back(PrefillItem{x.seq, x.kv_head, x.qtile, t0, std::min(x.tile_end, t0 + per), n_parts++, 0, 0});
        const int32_t ql = cu_q[x.seq + 1] - cu_q[x.seq];
        citems.push_back(CombineItem{part0, k, cu_q[x.seq] + x.qtile * rows, std::min(rows, ql - x.qtile * rows),
                                     x.kv_head * G, G, 0, 0});
        max_cost = std::max<int64_t>(max_cost, per);
      } else {
        expanded.push_back(x);
        max_cost = std::max(max_cost, cost);
      }
    }
    items.swap(expanded);
  }
  // Order: longest first (the persistent workgroups take the list in order).
  // Order 1 cuts the list into eight cost-balanced runs grouped by head, sorts
  // each longest first and interleaves them (item x of run k at 8x + k).
  auto lpt_sort = [&](std::vector<PrefillItem> &v) {
    std::vector<int32_t> &cnt = c->scratch_cnt;
    cnt.assign(static_cast<size_t>(max_cost) + 2, 0);
    for (const PrefillItem &x : v) cnt[static_cast<size_t>(max_cost - (x.tile_end - x.tile_begin))]++;
    int32_t acc = 0;
    for (int32_t &cv : cnt) {
      int32_t t = cv;
      cv = acc;
      acc += t;
    }
    std::vector<PrefillItem> sorted(v.size());
    for (const PrefillItem &x : v) sorted[static_cast<size_t>(cnt[static_cast<size_t>(max_cost - (x.tile_end - x.tile_begin))]++)] = x;
    v.swap(sorted);
  };
  if (c->prefill_order == 1 && items.size() > static_cast<size_t>(kXcds)) {
    int64_t tot = 0;
    for (const PrefillItem &x : items) tot += x.tile_end - x.tile_begin;
    std::vector<PrefillItem> q[kXcds];
    int64_t prefix = 0;
    for (const PrefillItem &x : items) {
      const int64_t cost = x.tile_end - x.tile_begin;
      const int64_t xcd = std::min<int64_t>(kXcds - 1, (2 * prefix + cost) * kXcds / (2 * std::max<int64_t>(tot, 1)));
      q[xcd].push_back(x);
      prefix += cost;
    }
    size_t n_q = 0;
    for (auto &v : q) {
      lpt_sort(v);
      n_q = std::max(n_q, v.size());
    }
    items.clear();
    for (size_t j = 0; j < n_q; ++j)
      for (int x = 0; x < kXcds; ++x)
        if (j < q[x].size()) items.push_back(q[x][j]);
  } else {
    lpt_sort(items);
  }
  const int32_t n_wgs = static_cast<int32_t>(std::min<int64_t>(
      static_cast<int64_t>(items.size()), std::max<int64_t>(1, static_cast<int64_t>(c->num_cus) * wg_per_cu)));
  std::vector<int32_t> &wg_off = c->scratch_wg;
  wg_off.assign(static_cast<size_t>(n_wgs) + 1, 0);
  if (c->prefill_kernel == kPrefillTwoGroup && n_wgs > 0) {
    // The two-group kernel runs a fixed list per workgroup: longest first,
    // each item to the least loaded workgroup (cost = tiles plus a constant
    // for the item's start and output).
    std::vector<int64_t> &cost = c->scratch_cost;
    cost.resize(items.size());
    for (size_t i = 0; i < items.size(); ++i) cost[i] = (items[i].tile_end - items[i].tile_begin) + kItemCostTiles;
    balance_items(cost, n_wgs, &c->scratch_owner, &wg_off, &c->scratch_order);
    std::vector<PrefillItem> grouped(items.size());
    for (size_t j = 0; j < items.size(); ++j) grouped[j] = items[static_cast<size_t>(c->scratch_order[j])];
    items.swap(grouped);
  }

  const SeqTables tl = seq_tables_layout(c, layer, n_seqs, seq_ids);
  pp->tl = tl;
  pp->tbytes = align_up(tl.bytes, 16);
  pp->ibytes = align_up(sizeof(PrefillItem) * items.size(), 16);
  pp->cbytes = align_up(sizeof(CombineItem) * citems.size(), 16);
  pp->wbytes = align_up(sizeof(int32_t) * wg_off.size(), 16);
  pp->bytes = pp->tbytes + pp->ibytes + pp->cbytes + 16 + pp->wbytes;
  pp->n_items = static_cast<int32_t>(items.size());
  pp->n_parts = n_parts;
  pp->n_wgs = n_wgs;
  out->assign(pp->bytes, 0);
  std::vector<int32_t> qs(n_seqs), ql(n_seqs);
  for (int32_t b = 0; b < n_seqs; ++b) {
    qs[b] = cu_q[b];
    ql[b] = cu_q[b + 1] - cu_q[b];
  }
  write_seq_tables(c, layer, n_seqs, seq_ids, qs.data(), ql.data(), tl, out->data());
  std::memcpy(out->data() + pp->tbytes, items.data(), sizeof(PrefillItem) * items.size());
  if (!citems.empty())
    std::memcpy(out->data() + pp->tbytes + pp->ibytes, citems.data(), sizeof(CombineItem) * citems.size());
  std::memcpy(out->data() + pp->tbytes + pp->ibytes + pp->cbytes + 16, wg_off.data(), sizeof(int32_t) * wg_off.size());
}

RopeArgs rope_args(const segkv_ctx *c, const SeqTables &t, const char *tables) {
  RopeArgs r;
  r.tables = reinterpret_cast<const float *>(tables + t.rope_off);
  r.lo = c->D - c->rope_dims;
  r.half = c->rope_dims / 2;
  r.style = c->rope_style;
  r.pad = 0;
  return r;
}

// Upper bounds of one call's tables and partials (bytes), for batches of at
// most max_seqs sequences and Q query tokens, with at most num_pages page ids
// listed and the automatic prefill split.  The counts follow the planners:
//   prefill  items per (sequence, KV head) = ceil(q_b / rows), so at most
//            Hkv (ceil(Q / rows) + S) unsplit items; an item is split only
//            when it exceeds total / slots tiles, so at most slots items are
//            split, into at most 2 slots parts;
//   decode   one piece per segment plus one per share boundary (slots shares);
//   scores   one partial row per visible (query tile, key tile) pair of an
//            item: tile counts grow with the query tile's index for a global
//            head and stop at the window for a local one.  The elementwise
//            largest tile counts are those of one sequence of all the
//            batch's query tiles.
struct WsBound {
  size_t tables = 0;  // largest tables of a prefill, decode or top-k call (staging room)
  size_t total = 0;   // largest tables + partials of any call
};

WsBound workspace_bound(const segkv_config *cfg, int64_t Q, int64_t slots) {
  const int64_t S = cfg->max_seqs, Hkv = cfg->num_kv_heads, D = cfg->head_dim;
  const int64_t G = cfg->num_q_heads / cfg->num_kv_heads;
  const int64_t rows = std::max<int64_t>(1, kPrefillRows / G);
  const int64_t nseg = S * Hkv;
  const size_t seq_tables = align_up(sizeof(SeqDesc) * S, 16) + align_up(sizeof(SegDesc) * nseg, 16) +
                            align_up(sizeof(int32_t) * static_cast<size_t>(cfg->num_pages), 16) +
                            sizeof(float) * 2 * D * nseg;
  auto with_parts = [](size_t t, size_t p) { return align_up(align_up(t, 16), 256) + p; };
  WsBound b;
  // prefill: the larger of the default item shape (kPrefillRows rows, slots
  // workgroups) and the two-workgroup variant's (kPrefillDuoRows rows, twice
  // the workgroups); partial slots hold kPrefillRows rows either way
  const int64_t nq_tiles = ceil_div(Q, rows) + S;
  size_t p_tables = 0, p_part = 0;
  for (int shape = 0; shape < 2; ++shape) {
    const int64_t r = shape ? std::max<int64_t>(1, kPrefillDuoRows / G) : rows;
    const int64_t sl = shape ? slots / kPrefillWgPerCu * kPrefillDuoWgPerCu : slots;
    const int64_t items = Hkv * (ceil_div(Q, r) + S);
    const int64_t parts = 2 * sl;
    const size_t t = align_up(seq_tables, 16) + align_up(sizeof(PrefillItem) * (items + parts), 16) +
                     align_up(sizeof(CombineItem) * std::min(items, sl), 16) + 16 +
                     align_up(sizeof(int32_t) * static_cast<size_t>(sl + 1), 16);
    const size_t pp = static_cast<size_t>(parts) * kPrefillRows * (D + 1) * sizeof(float);
    p_tables = std::max(p_tables, t);
    p_part = std::max(p_part, pp);
  }
  const int64_t base_items = Hkv * nq_tiles;
  // decode: one piece per (segment, block of kDecodeCols query heads) plus one per share boundary
  const int64_t nvseg = nseg * ceil_div(G, kDecodeCols);
  const int64_t pieces = nvseg + slots;
  const size_t d_tables = align_up(seq_tables, 16) + align_up(sizeof(DecodeItem) * pieces, 16) +
                          align_up(sizeof(int32_t) * (slots + 1), 16) + sizeof(CombineItem) * nvseg;
  const size_t d_part = static_cast<size_t>(pieces) * kDecodeCols * (D + 1) * sizeof(float);
  // top-k (the tables of max_seqs sequences)
  const size_t k_tables = align_up(sizeof(int32_t) * (S + 1), 16) + 2 * align_up(sizeof(int32_t) * S, 16);
  // token scores: worst layer
  int64_t part_rows = 0;
  for (int32_t layer = 0; layer < cfg->num_layers; ++layer) {
    int64_t r = 0;
    for (int64_t g = 0; g < Hkv; ++g) {
      const int64_t w = cfg->head_window[layer * Hkv + g];
      for (int64_t qt = 0; qt < nq_tiles; ++qt) {
        int64_t t = ((qt + 1) * rows - 1) / kTileKeys + 2;
        if (w > 0) t = std::min<int64_t>(t, (rows + w - 2) / kTileKeys + 2);
        r += t;
      }
    }
    part_rows = std::max(part_rows, r);
  }
  const int64_t srows = ceil_div(Q, kTileKeys) + 2 * S;
  // items are cut into pieces of at least kMinSplitTiles tiles
  const int64_t cut_items = base_items + ceil_div(part_rows, kMinSplitTiles);
  const size_t s_tables = align_up(seq_tables, 16) + align_up(sizeof(PrefillItem) * cut_items, 16) +
                          align_up(sizeof(ScoreRow) * srows, 16) + align_up(sizeof(int32_t) * part_rows, 16) + 16;
  const size_t s_part = static_cast<size_t>(std::max<int64_t>(part_rows, 1)) * kTileKeys * sizeof(float);
  b.tables = std::max({p_tables, d_tables, k_tables});
  b.total = std::max({with_parts(p_tables, p_part), with_parts(d_tables, d_part), with_parts(s_tables, s_part),
                      align_up(k_tables, 256)});
  return b;
}

// Resident workgroup slots of the current device (one prefill or decode
// workgroup per CU); the bound assumes 256 when no device answers.
int64_t device_slots() {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                             hipSuccess || cus <= 0)
    return 256;
  return std::max<int64_t>(cus, 1) * std::max(kPrefillWgPerCu, kDecodeWgPerCu);
}

constexpr int32_t kDefaultMaxBatchQ = 16384;

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================

extern "C" {

int segkv_create(const segkv_config *cfg, segkv_ctx **out) {
  g_create_error.clear();
  auto bad = [](int code, const char *msg) {
    g_create_error = msg;
    return code;
  };
  if (!out) return bad(SEGKV_E_INVAL, "out is NULL");
  *out = nullptr;
  if (!cfg) return bad(SEGKV_E_INVAL, "cfg is NULL");
  if (cfg->num_layers <= 0) return bad(SEGKV_E_INVAL, "num_layers must be > 0");
  if (cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0) return bad(SEGKV_E_INVAL, "head counts must be > 0");
  if (cfg->num_q_heads % cfg->num_kv_heads)
    return bad(SEGKV_E_INVAL, "num_q_heads must be a multiple of num_kv_heads");
  if (cfg->num_q_heads / cfg->num_kv_heads > kPrefillRows)
    return bad(SEGKV_E_INVAL, "num_q_heads / num_kv_heads must be <= 128");
  if (cfg->head_dim != 64 && cfg->head_dim != 128) return bad(SEGKV_E_INVAL, "head_dim must be 64 or 128");
  if (cfg->page_size != 16 && cfg->page_size != 32 && cfg->page_size != 64)
    return bad(SEGKV_E_INVAL, "page_size must be 16, 32 or 64");
  if (cfg->max_seqs <= 0) return bad(SEGKV_E_INVAL, "max_seqs must be > 0");
  if (cfg->num_pages <= 0 || cfg->num_pages > std::numeric_limits<int32_t>::max())
    return bad(SEGKV_E_INVAL, "num_pages must be in [1, 2^31)");
  if (!cfg->head_window) return bad(SEGKV_E_INVAL, "head_window is NULL");
  if ((cfg->k_pool == nullptr) != (cfg->v_pool == nullptr))
    return bad(SEGKV_E_INVAL, "k_pool and v_pool must both be set or both be NULL");
  if (!(cfg->softmax_scale >= 0.f) || std::isinf(cfg->softmax_scale))
    return bad(SEGKV_E_INVAL, "softmax_scale must be finite and >= 0");
  if (!(cfg->rope_theta >= 0.f) || std::isinf(cfg->rope_theta) || (cfg->rope_theta > 0.f && cfg->rope_theta <= 1.f))
    return bad(SEGKV_E_INVAL, "rope_theta must be 0 (default) or a finite value > 1");
  if (cfg->rope_style != 0 && cfg->rope_style != 1)
    return bad(SEGKV_E_INVAL, "rope_style must be 0 (rotate-half) or 1 (interleaved)");
  if (cfg->rope_dims != 0 && (cfg->rope_dims < 16 || cfg->rope_dims > cfg->head_dim || cfg->rope_dims % 16))
    return bad(SEGKV_E_INVAL, "rope_dims must be 0 or a multiple of 16 in [16, head_dim]");
  size_t nwin = static_cast<size_t>(cfg->num_layers) * cfg->num_kv_heads;
  for (size_t i = 0; i < nwin; ++i)
    if (cfg->head_window[i] < 0) return bad(SEGKV_E_INVAL, "head_window entries must be >= 0");
  if (cfg->max_batch_q_tokens < 0) return bad(SEGKV_E_INVAL, "max_batch_q_tokens must be >= 0");
  if (cfg->workspace && reinterpret_cast<uintptr_t>(cfg->workspace) % 256)
    return bad(SEGKV_E_INVAL, "workspace must be 256-byte aligned");
  if (cfg->workspace && cfg->workspace_bytes == 0) return bad(SEGKV_E_INVAL, "workspace given with 0 bytes");

  segkv_ctx *c = new (std::nothrow) segkv_ctx();
  if (!c) return bad(SEGKV_E_NOMEM, "out of host memory");
  c->L = cfg->num_layers;
  c->Hq = cfg->num_q_heads;
  c->Hkv = cfg->num_kv_heads;
  c->G = c->Hq / c->Hkv;
  c->D = cfg->head_dim;
  c->P = cfg->page_size;
  c->S = cfg->max_seqs;
  c->num_pages = cfg->num_pages;
  c->scale = cfg->softmax_scale > 0.f ? cfg->softmax_scale : 1.0f / std::sqrt(static_cast<float>(cfg->head_dim));
  c->window.assign(cfg->head_window, cfg->head_window + nwin);
  c->rope_theta = cfg->rope_theta > 0.f ? static_cast<double>(cfg->rope_theta) : 10000.0;
  c->rope_style = cfg->rope_style;
  c->rope_dims = cfg->rope_dims ? cfg->rope_dims : cfg->head_dim;
  c->k_pool = static_cast<uint16_t *>(cfg->k_pool);
  c->v_pool = static_cast<uint16_t *>(cfg->v_pool);
  c->stream = static_cast<hipStream_t>(cfg->stream);
  c->planning = cfg->k_pool == nullptr;
  c->max_q = cfg->max_batch_q_tokens ? cfg->max_batch_q_tokens : kDefaultMaxBatchQ;
  try {
    c->segs.resize(static_cast<size_t>(c->L) * c->S * c->Hkv);
    c->seq_layer.resize(static_cast<size_t>(c->L) * c->S);
    c->free_list.resize(static_cast<size_t>(c->num_pages));
    c->refcnt.assign(static_cast<size_t>(c->num_pages), 0);
  } catch (...) {
    delete c;
    return bad(SEGKV_E_NOMEM, "out of host memory for allocator state");
  }
  // back() is handed out first: index order for seed 0, else a seeded shuffle.
  for (int64_t i = 0; i < c->num_pages; ++i) c->free_list[static_cast<size_t>(i)] = static_cast<int32_t>(c->num_pages - 1 - i);
  if (cfg->page_order_seed) {
    std::mt19937_64 rng(cfg->page_order_seed);
    for (size_t i = c->free_list.size(); i > 1; --i) {
      size_t j = static_cast<size_t>(rng() % i);
      std::swap(c->free_list[i - 1], c->free_list[j]);
    }
  }
  if (!c->planning) {
    int dev = 0;
    hipError_t e0 = hipGetDevice(&dev);
    if (e0 == hipSuccess) e0 = hipDeviceGetAttribute(&c->num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e0 != hipSuccess) {
      g_create_error = std::string("hipDeviceGetAttribute: ") + hipGetErrorString(e0);
      segkv_destroy(c);
      return SEGKV_E_DEVICE;
    }
    for (int i = 0; i < kStages / kStageGroup; ++i) {
      hipError_t e = hipEventCreateWithFlags(&c->stage_ev[i], hipEventDisableTiming);
      if (e != hipSuccess) {
        g_create_error = std::string("hipEventCreate: ") + hipGetErrorString(e);
        segkv_destroy(c);
        return SEGKV_E_DEVICE;
      }
    }
    // Workspace: the caller's, else allocated here once.  Staging buffers are
    // sized here for the largest prefill, decode or top-k tables of
    // max_batch_q_tokens, so calls in that range allocate nothing.
    const WsBound wb = workspace_bound(cfg, c->max_q, static_cast<int64_t>(c->num_cus) * kPrefillWgPerCu);
    if (cfg->workspace) {
      c->ws = static_cast<char *>(cfg->workspace);
      c->ws_bytes = cfg->workspace_bytes;
    } else {
      c->ws_bytes = cfg->workspace_bytes ? cfg->workspace_bytes : wb.total;
      hipError_t e = hipMalloc(reinterpret_cast<void **>(&c->ws), c->ws_bytes);
      if (e != hipSuccess) {
        g_create_error = std::string("hipMalloc(workspace): ") + hipGetErrorString(e);
        c->ws = nullptr;
        segkv_destroy(c);
        return SEGKV_E_NOMEM;
      }
      c->ws_owned = true;
    }
    {
      void *p = nullptr;
      hipError_t e = scratch_address(&p);
      if (e != hipSuccess) {
        g_create_error = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
        segkv_destroy(c);
        return SEGKV_E_DEVICE;
      }
      c->fixed_scratch = static_cast<char *>(p);
    }
    c->pre_room = std::max(c->pre_room, std::min(wb.tables, c->ws_bytes));
    for (int i = 0; i < kStages; ++i) {
      const int rc = ensure_stage(c, i, align_up(wb.tables, 16) + c->pre_room);
      if (rc) {
        g_create_error = c->err;
        segkv_destroy(c);
        return rc;
      }
    }
  }
  *out = c;
  return SEGKV_OK;
}

void segkv_destroy(segkv_ctx *c) {
  if (!c) return;
  if (!c->planning) {
    (void)hipStreamSynchronize(c->stream);
    for (const TimedLaunch &t : c->pending) {
      (void)hipEventDestroy(t.start);
      (void)hipEventDestroy(t.stop);
    }
    for (hipEvent_t e : c->event_pool) (void)hipEventDestroy(e);
    for (int i = 0; i < kStages / kStageGroup; ++i)
      if (c->stage_ev[i]) (void)hipEventDestroy(c->stage_ev[i]);
    for (int i = 0; i < kStages; ++i)
      if (c->h_stage[i]) (void)hipHostFree(c->h_stage[i]);
    if (c->ws_owned && c->ws) (void)hipFree(c->ws);
  }
  delete c;
}

const char *segkv_last_error(const segkv_ctx *c) { return c ? c->err.c_str() : g_create_error.c_str(); }

size_t segkv_workspace_bytes(const segkv_config *cfg, int32_t max_batch_q_tokens) {
  if (!cfg || max_batch_q_tokens < 0 || cfg->num_layers <= 0 || cfg->num_q_heads <= 0 || cfg->num_kv_heads <= 0 ||
      cfg->num_q_heads % cfg->num_kv_heads || (cfg->head_dim != 64 && cfg->head_dim != 128) || cfg->max_seqs <= 0 ||
      cfg->num_pages <= 0 || cfg->num_pages > std::numeric_limits<int32_t>::max() || !cfg->head_window)
    return 0;
  return workspace_bound(cfg, max_batch_q_tokens, device_slots()).total;
}

int64_t segkv_free_pages(const segkv_ctx *c) {
  if (!c) return SEGKV_E_INVAL;
  return static_cast<int64_t>(c->free_list.size());
}

int segkv_page_table(const segkv_ctx *cc, int32_t layer, int32_t seq_id, int32_t kv_head, int32_t *first_token,
                     int32_t *kv_len, int32_t *n_pages, int32_t *page_ids, int32_t cap) {
  segkv_ctx *c = const_cast<segkv_ctx *>(cc);
  if (!c) return SEGKV_E_INVAL;
  if (layer < 0 || layer >= c->L) return c->fail(SEGKV_E_RANGE, "layer %d out of range", layer);
  if (seq_id < 0 || seq_id >= c->S) return c->fail(SEGKV_E_RANGE, "seq id %d out of range", seq_id);
  if (kv_head < 0 || kv_head >= c->Hkv) return c->fail(SEGKV_E_RANGE, "kv head %d out of range", kv_head);
  if (cap < 0) return c->fail(SEGKV_E_INVAL, "cap < 0");
  const Segment &s = c->seg(layer, seq_id, kv_head);
  if (first_token) *first_token = s.first_token;
  if (kv_len) *kv_len = c->sl(layer, seq_id).kv_len;
  if (n_pages) *n_pages = s.n_live();
  if (page_ids) std::memcpy(page_ids, s.live(), sizeof(int32_t) * std::min<int32_t>(cap, s.n_live()));
  return SEGKV_OK;
}

int segkv_set_relocation(segkv_ctx *c, int32_t seq_id, const int32_t *deltas) {
  if (!c) return SEGKV_E_INVAL;
  if (seq_id < 0 || seq_id >= c->S) return c->fail(SEGKV_E_RANGE, "seq id %d out of range", seq_id);
  for (int32_t layer = 0; layer < c->L; ++layer)
    for (int32_t g = 0; g < c->Hkv; ++g)
      c->seg(layer, seq_id, g).delta = deltas ? deltas[static_cast<size_t>(layer) * c->Hkv + g] : 0;
  return SEGKV_OK;
}

int segkv_fork(segkv_ctx *c, int32_t src_seq, int32_t dst_seq) {
  if (!c) return SEGKV_E_INVAL;
  if (src_seq < 0 || src_seq >= c->S || dst_seq < 0 || dst_seq >= c->S)
    return c->fail(SEGKV_E_RANGE, "seq id out of range (src %d, dst %d)", src_seq, dst_seq);
  if (src_seq == dst_seq) return c->fail(SEGKV_E_INVAL, "fork needs two different sequences");
  for (int32_t layer = 0; layer < c->L; ++layer) {
    if (c->sl(layer, dst_seq).kv_len != 0) return c->fail(SEGKV_E_STATE, "fork target %d is not empty", dst_seq);
    for (int32_t g = 0; g < c->Hkv; ++g)
      if (c->seg(layer, dst_seq, g).n_live() != 0) return c->fail(SEGKV_E_STATE, "fork target %d holds pages", dst_seq);
  }
  for (int32_t layer = 0; layer < c->L; ++layer) {
    c->sl(layer, dst_seq) = c->sl(layer, src_seq);
    for (int32_t g = 0; g < c->Hkv; ++g) {
      const Segment &from = c->seg(layer, src_seq, g);
      Segment &to = c->seg(layer, dst_seq, g);
      to.first_token = from.first_token;
      to.delta = from.delta;
      to.head = 0;
      to.pages.assign(from.live(), from.live() + from.n_live());
      for (int32_t id : to.pages) c->refcnt[static_cast<size_t>(id)]++;
    }
  }
  return SEGKV_OK;
}

int segkv_release(segkv_ctx *c, int32_t seq_id) {
  if (!c) return SEGKV_E_INVAL;
  if (seq_id < 0 || seq_id >= c->S) return c->fail(SEGKV_E_RANGE, "seq id %d out of range", seq_id);
  for (int32_t layer = 0; layer < c->L; ++layer) {
    for (int32_t g = 0; g < c->Hkv; ++g) {
      Segment &s = c->seg(layer, seq_id, g);
      for (int32_t i = 0; i < s.n_live(); ++i) c->drop_page(s.live()[i]);
      s.pages.clear();
      s.head = 0;
      s.first_token = 0;
      s.delta = 0;
    }
    c->sl(layer, seq_id) = SeqLayer{};
  }
  return SEGKV_OK;
}

int segkv_append_pages(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const int32_t *cu_new,
                       const int32_t *n_query, const void *k_new, const void *v_new) {
  if (!c) return SEGKV_E_INVAL;
  int rc = check_layer_seqs(c, layer, n_seqs, seq_ids);
  if (rc) return rc;
  if (n_seqs == 0) return SEGKV_OK;
  if (!cu_new || !n_query) return c->fail(SEGKV_E_INVAL, "cu_new / n_query is NULL");
  if (cu_new[0] != 0) return c->fail(SEGKV_E_INVAL, "cu_new[0] must be 0");
  for (int32_t b = 0; b < n_seqs; ++b) {
    int32_t n = cu_new[b + 1] - cu_new[b];
    if (cu_new[b + 1] < cu_new[b]) return c->fail(SEGKV_E_INVAL, "cu_new must be non-decreasing");
    if (n_query[b] < 0 || n_query[b] > n)
      return c->fail(SEGKV_E_INVAL, "n_query[%d] = %d must be in [0, %d]", b, n_query[b], n);
    if (static_cast<int64_t>(c->sl(layer, seq_ids[b]).kv_len) + n > std::numeric_limits<int32_t>::max() / 2)
      return c->fail(SEGKV_E_INVAL, "sequence length overflow");
    for (int32_t b2 = 0; b2 < b; ++b2)
      if (seq_ids[b2] == seq_ids[b]) return c->fail(SEGKV_E_INVAL, "duplicate seq id %d in one append", seq_ids[b]);
  }
  const int32_t total_new = cu_new[n_seqs];
  if (c->planning) {
    if (k_new || v_new) return c->fail(SEGKV_E_STATE, "planning-only context takes k_new = v_new = NULL");
  } else if (total_new > 0 && (!k_new || !v_new)) {
    return c->fail(SEGKV_E_INVAL, "k_new / v_new is NULL");
  }

  // Plan: per (b, g) the new segment start, pages dropped, kept and added,
  // and whether the kept tail page is shared with a fork and must be copied
  // before the new tokens are written into it.
  const int32_t P = c->P;
  constexpr int kPlan = 5;
  std::vector<int32_t> &plan = c->scratch_i32;  // [n_seqs*Hkv][5]: new_first, n_drop, n_keep, n_add, cow
  plan.assign(static_cast<size_t>(n_seqs) * c->Hkv * kPlan, 0);
  int64_t need = 0, freed = 0;
  std::vector<std::pair<int32_t, int32_t>> shared_drops;  // dropped pages that other segments also hold
  for (int32_t b = 0; b < n_seqs; ++b) {
    const SeqLayer &s = c->sl(layer, seq_ids[b]);
    const int32_t new_kv = s.kv_len + (cu_new[b + 1] - cu_new[b]);
    for (int32_t g = 0; g < c->Hkv; ++g) {
      const Segment &sg = c->seg(layer, seq_ids[b], g);
      const int32_t w = c->win(layer, g);
      int32_t new_first = sg.first_token;
      if (w > 0) new_first = std::max(new_first, local_segment_start(new_kv, n_query[b], w, P));
      int32_t n_drop = std::min<int32_t>(sg.n_live(), (new_first - sg.first_token) / P);
      int32_t n_keep = sg.n_live() - n_drop;
      int32_t n_total = new_kv > new_first ? static_cast<int32_t>(ceil_div(new_kv - new_first, P)) : 0;
      int32_t n_add = std::max(0, n_total - n_keep);
      // The first new token lands in kept page (tok_lo - new_first) / P; when
      // that is the kept tail and a fork also holds it, copy it first.
      const int32_t tok_lo = std::max(s.kv_len, new_first);
      int32_t cow = 0;
      if (n_keep > 0 && tok_lo < new_kv && (tok_lo - new_first) / P == n_keep - 1 &&
          c->refcnt[static_cast<size_t>(sg.live()[n_drop + n_keep - 1])] > 1)
        cow = 1;
      int32_t *pl = &plan[(static_cast<size_t>(b) * c->Hkv + g) * kPlan];
      pl[0] = new_first;
      pl[1] = n_drop;
      pl[2] = n_keep;
      pl[3] = n_add;
      pl[4] = cow;
      need += n_add + cow;
      for (int32_t i = 0; i < n_drop; ++i) {
        const int32_t id = sg.live()[i];
        if (c->refcnt[static_cast<size_t>(id)] == 1) ++freed;
        else shared_drops.emplace_back(id, 1);
      }
    }
  }
  if (!shared_drops.empty()) {  // shared pages dropped by every holder in this call are freed too
    std::sort(shared_drops.begin(), shared_drops.end());
    for (size_t i = 0; i < shared_drops.size();) {
      size_t j = i;
      while (j < shared_drops.size() && shared_drops[j].first == shared_drops[i].first) ++j;
      if (static_cast<int64_t>(j - i) == c->refcnt[static_cast<size_t>(shared_drops[i].first)]) ++freed;
      i = j;
    }
  }
  if (need > static_cast<int64_t>(c->free_list.size()) + freed)
    return c->fail(SEGKV_E_NOMEM, "page pool exhausted: need %lld pages, %lld free (+%lld reclaimable)",
                   static_cast<long long>(need), static_cast<long long>(c->free_list.size()),
                   static_cast<long long>(freed));

  // Count scatter items (pages touched) and size the upload before changing state.
  int64_t n_items = 0;
  if (!c->planning) {
    for (int32_t b = 0; b < n_seqs; ++b) {
      const SeqLayer &s = c->sl(layer, seq_ids[b]);
      const int32_t new_kv = s.kv_len + (cu_new[b + 1] - cu_new[b]);
      for (int32_t g = 0; g < c->Hkv; ++g) {
        const int32_t *pl = &plan[(static_cast<size_t>(b) * c->Hkv + g) * kPlan];
        int32_t tok_lo = std::max(s.kv_len, pl[0]);
        if (tok_lo >= new_kv) continue;
        n_items += (new_kv - 1 - pl[0]) / P - (tok_lo - pl[0]) / P + 1;
      }
    }
  }
  // When the queries are a prefill chunk (some sequence has more than one),
  // the tables of their prefill ride along: built after the state change
  // into room kept behind the scatter items, and copied to the device by the
  // scatter launch, so that the prefill call needs no upload of its own.
  int64_t n_queries = 0;
  for (int32_t b = 0; b < n_seqs; ++b) n_queries += n_query[b];
  const bool prestage = !c->planning && n_items > 0 && n_queries > n_seqs;
  char *stage = nullptr;
  int slot = 0;
  const size_t bytes = align_up(sizeof(ScatterItem) * static_cast<size_t>(n_items), 16);
  if (!c->planning && n_items > 0) {
    rc = acquire_stage(c, bytes + (prestage ? c->pre_room : 0), &stage, &slot);
    if (rc) return rc;
  }

  // Commit in two phases.  First every trim of the batch returns its pages,
  // so that the check above (which counted them as available) holds for
  // each allocation that follows, whatever the order of growing and
  // trimming heads and sequences.  Then shared tails are copied, pages are
  // allocated and scatter work is recorded.  A copied page's reference is
  // dropped only after every allocation of the call, so a page that this
  // launch reads as a copy source is never handed out (and written) by the
  // same launch.
  for (int32_t b = 0; b < n_seqs; ++b) {
    for (int32_t g = 0; g < c->Hkv; ++g) {
      Segment &sg = c->seg(layer, seq_ids[b], g);
      const int32_t *pl = &plan[(static_cast<size_t>(b) * c->Hkv + g) * kPlan];
      for (int32_t i = 0; i < pl[1]; ++i) c->drop_page(sg.live()[i]);
      sg.drop_front(pl[1]);
      sg.first_token = pl[0];
    }
  }
  ScatterItem *items = reinterpret_cast<ScatterItem *>(stage);
  int64_t it = 0;
  std::vector<int32_t> &cow_src = c->scratch_release;
  cow_src.clear();
  for (int32_t b = 0; b < n_seqs; ++b) {
    SeqLayer &s = c->sl(layer, seq_ids[b]);
    const int32_t old_kv = s.kv_len;
    const int32_t new_kv = old_kv + (cu_new[b + 1] - cu_new[b]);
    for (int32_t g = 0; g < c->Hkv; ++g) {
      Segment &sg = c->seg(layer, seq_ids[b], g);
      const int32_t *pl = &plan[(static_cast<size_t>(b) * c->Hkv + g) * kPlan];
      int32_t cow_from = -1;
      if (pl[4]) {
        int32_t &tail = sg.pages[sg.head + static_cast<size_t>(pl[2] - 1)];
        cow_from = tail;
        cow_src.push_back(tail);
        tail = c->take_page();
      }
      for (int32_t i = 0; i < pl[3]; ++i) sg.pages.push_back(c->take_page());
      if (c->planning) continue;
      const int32_t tok_lo = std::max(old_kv, pl[0]);
      if (tok_lo >= new_kv) continue;
      const int32_t first_idx = (tok_lo - pl[0]) / P;
      const int32_t last_idx = (new_kv - 1 - pl[0]) / P;
      for (int32_t pi = first_idx; pi <= last_idx; ++pi) {
        const int32_t ps = pl[0] + pi * P;
        const int32_t t0 = std::max(ps, tok_lo);
        const int32_t t1 = std::min(ps + P, new_kv);
        ScatterItem &si = items[it++];
        si.page_id = sg.live()[pi];
        si.kv_head = g;
        si.slot_begin = t0 - ps;
        si.slot_end = t1 - ps;
        si.src_row = cu_new[b] + (t0 - old_kv);
        const bool copied = pl[4] && pi == pl[2] - 1;
        si.zero_tail = pi >= pl[2] || copied ? 1 : 0;
        si.copy_from = copied ? cow_from : -1;
        si.pad1 = 0;
      }
    }
    s.kv_len = new_kv;
    s.pending_from = new_kv - n_query[b];
  }
  for (int32_t id : cow_src) c->drop_page(id);
  if (c->planning || n_items == 0) return SEGKV_OK;

  ScatterArgs a;
  a.k_new = static_cast<const uint16_t *>(k_new);
  a.v_new = static_cast<const uint16_t *>(v_new);
  a.k_pool = c->k_pool;
  a.v_pool = c->v_pool;
  // The scatter work list is read straight from the pinned staging buffer
  // (one 32-byte item per workgroup), so the append needs no upload.
  a.items = reinterpret_cast<const ScatterItem *>(c->h_stage_dev[slot]);
  a.num_kv_heads = c->Hkv;
  a.copy_src = nullptr;
  a.copy_dst = nullptr;
  a.copy_n16 = 0;
  a.copy_wgs = 0;
  bool staged = false;
  if (prestage) {
    std::vector<int32_t> cu_q(static_cast<size_t>(n_seqs) + 1, 0);
    for (int32_t b = 0; b < n_seqs; ++b) cu_q[b + 1] = cu_q[b] + n_query[b];
    PrefillPlan pp;
    build_prefill_plan(c, layer, n_seqs, seq_ids, cu_q.data(), &pp, &c->plan_buf);
    if (bytes + pp.bytes <= c->h_stage_cap[slot] && pp.bytes <= c->ws_bytes) {
      std::memcpy(stage + bytes, c->plan_buf.data(), pp.bytes);
      c->pre_buf.swap(c->plan_buf);
      a.copy_src = reinterpret_cast<const uint4 *>(c->h_stage_dev[slot] + bytes);
      a.copy_dst = reinterpret_cast<uint4 *>(c->ws);
      a.copy_n16 = static_cast<int32_t>(pp.bytes / 16);
      a.copy_wgs = static_cast<int32_t>(std::min<size_t>(kScatterCopyWgs, ceil_div(pp.bytes / 16, kScatterThreads)));
      staged = true;
    }
    c->pre_room = std::max(c->pre_room, std::min(pp.bytes, c->ws_bytes));  // the next append keeps room enough
  }
  c->pre_valid = false;
  TimedLaunch t{};
  rc = timed_begin(c, &t, SEGKV_KERNEL_SCATTER);
  if (rc) return rc;
  hipError_t e = launch_scatter(a, static_cast<int>(n_items), c->D, c->P, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "scatter launch");
  c->pre_valid = staged;
  return timed_end(c, &t);
}

int segkv_prefill(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const int32_t *cu_q,
                  const void *q, void *o, float *lse) {
  if (!c) return SEGKV_E_INVAL;
  if (c->planning) return c->fail(SEGKV_E_STATE, "prefill needs device pools (planning-only context)");
  int rc = check_layer_seqs(c, layer, n_seqs, seq_ids);
  if (rc) return rc;
  if (n_seqs == 0) return SEGKV_OK;
  if (!cu_q) return c->fail(SEGKV_E_INVAL, "cu_q is NULL");
  if (cu_q[0] != 0) return c->fail(SEGKV_E_INVAL, "cu_q[0] must be 0");
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int32_t ql = cu_q[b + 1] - cu_q[b];
    const SeqLayer &s = c->sl(layer, seq_ids[b]);
    if (ql < 0) return c->fail(SEGKV_E_INVAL, "cu_q must be non-decreasing");
    if (ql > s.kv_len) return c->fail(SEGKV_E_INVAL, "q_len %d > kv_len %d (seq %d)", ql, s.kv_len, seq_ids[b]);
    if (ql > 0 && s.kv_len - ql < s.pending_from)
      return c->fail(SEGKV_E_INVAL,
                     "seq %d: queries start at %d, before the earliest pending query %d declared at append",
                     seq_ids[b], s.kv_len - ql, s.pending_from);
  }
  const int32_t total_q = cu_q[n_seqs];
  if (total_q == 0) return SEGKV_OK;
  if (!q || !o) return c->fail(SEGKV_E_INVAL, "q / o is NULL");

  PrefillPlan pp;
  std::vector<char> &tables = c->plan_buf;
  build_prefill_plan(c, layer, n_seqs, seq_ids, cu_q, &pp, &tables);
  const int32_t n_parts = pp.n_parts;
  const size_t part_bytes = static_cast<size_t>(n_parts) * kPrefillRows * (c->D + 1) * sizeof(float);
  float *parts = nullptr;
  rc = carve(c, c->ws, c->ws_bytes, pp.bytes, part_bytes, &parts);
  if (rc) return rc;
  // The append that declared these queries may have put the same tables on
  // the device already (its scatter launch copies them).
  const bool staged = c->pre_valid && c->pre_buf.size() == pp.bytes &&
                      std::memcmp(c->pre_buf.data(), tables.data(), pp.bytes) == 0;
  if (!staged) {
    char *stage = nullptr;
    int slot = 0;
    rc = acquire_stage(c, pp.bytes, &stage, &slot);
    if (rc) return rc;
    std::memcpy(stage, tables.data(), pp.bytes);
    rc = upload(c, slot, pp.bytes, c->ws);
    if (rc) return rc;
  }
  c->pre_valid = false;  // this launch consumes the counters
  const SeqTables &tl = pp.tl;
  const size_t tbytes = pp.tbytes, ibytes = pp.ibytes, cbytes = pp.cbytes;
  const std::vector<CombineItem> &citems = c->scratch_citems;
  const int32_t G = c->G;
  const int32_t rows = prefill_item_rows(c) / G;

  PrefillArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.o = static_cast<uint16_t *>(o);
  a.lse = lse;
  a.k_pool = c->k_pool;
  a.v_pool = c->v_pool;
  a.seqs = reinterpret_cast<const SeqDesc *>(c->ws);
  a.segs = reinterpret_cast<const SegDesc *>(c->ws + tl.seg_off);
  a.page_ids = reinterpret_cast<const int32_t *>(c->ws + tl.pid_off);
  a.rope = rope_args(c, tl, c->ws);
  a.items = reinterpret_cast<const PrefillItem *>(c->ws + tbytes);
  a.part_o = parts;
  a.part_lse = parts ? parts + static_cast<size_t>(n_parts) * kPrefillRows * c->D : nullptr;
  a.num_q_heads = c->Hq;
  a.num_kv_heads = c->Hkv;
  a.group = G;
  a.rows_per_tile = rows;
  a.scale = c->scale;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  a.n_items = pp.n_items;
  a.counter = reinterpret_cast<int32_t *>(c->ws + tbytes + ibytes + cbytes);
  a.wg_items = reinterpret_cast<const int32_t *>(c->ws + tbytes + ibytes + cbytes + 16);
  const int n_wgs = pp.n_wgs;
  TimedLaunch t{};
  rc = timed_begin(c, &t, SEGKV_KERNEL_PREFILL);
  if (rc) return rc;
  hipError_t e = c->prefill_kernel == kPrefillDuo         ? launch_prefill_duo(a, n_wgs, c->D, c->P, c->stream)
                 : c->prefill_kernel == kPrefillPipelined ? launch_prefill_sp(a, n_wgs, c->D, c->P, c->stream)
                 : c->prefill_kernel == kPrefillTwoGroup ? launch_prefill_pp(a, n_wgs, c->D, c->P, c->stream)
                 : c->prefill_kernel == kPrefillWide   ? launch_prefill_wide(a, n_wgs, c->D, c->P, c->stream)
                                                       : launch_prefill(a, n_wgs, c->D, c->P, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "prefill launch");
  rc = timed_end(c, &t);
  if (rc) return rc;
  if (!citems.empty()) {
    CombineArgs ca;
    ca.part_o = a.part_o;
    ca.part_lse = a.part_lse;
    ca.items = reinterpret_cast<const CombineItem *>(c->ws + tbytes + ibytes);
    ca.o = static_cast<uint16_t *>(o);
    ca.lse = lse;
    ca.num_q_heads = c->Hq;
    ca.slot_rows = kPrefillRows;
    TimedLaunch t2{};
    rc = timed_begin(c, &t2, SEGKV_KERNEL_COMBINE);
    if (rc) return rc;
    e = launch_combine(ca, static_cast<int>(citems.size()), kPrefillRows, c->D, c->stream);
    if (e != hipSuccess) return c->device_fail(e, "combine launch");
    rc = timed_end(c, &t2);
    if (rc) return rc;
  }
  return SEGKV_OK;
}

}  // extern "C"

namespace {

// One-token decode with its tables at `base` and its partials after them,
// within cap bytes of device memory.
int decode_impl(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const void *q, void *o,
                float *lse, char *base, size_t cap, bool no_alloc) {
  if (!c) return SEGKV_E_INVAL;
  if (c->planning) return c->fail(SEGKV_E_STATE, "decode needs device pools (planning-only context)");
  int rc = check_layer_seqs(c, layer, n_seqs, seq_ids);
  if (rc) return rc;
  if (n_seqs == 0) return SEGKV_OK;
  if (!q || !o) return c->fail(SEGKV_E_INVAL, "q / o is NULL");
  for (int32_t b = 0; b < n_seqs; ++b) {
    const SeqLayer &s = c->sl(layer, seq_ids[b]);
    if (s.kv_len < 1) return c->fail(SEGKV_E_STATE, "seq %d is empty", seq_ids[b]);
    if (s.pending_from > s.kv_len - 1)
      return c->fail(SEGKV_E_INVAL, "seq %d: the last token was not appended as a query (n_query >= 1)", seq_ids[b]);
  }
  int32_t n_parts_total = 0;
  // Stream-K plan: the visible pages of all segments, in (sequence, KV head,
  // head block) order, are cut into equal contiguous shares, one per
  // workgroup (at most the GPU's resident decode workgroups, at least
  // min_pages pages each).  A work item takes up to kDecodeCols query heads
  // of a KV group; a larger group is NB blocks of them, each reading the
  // segment's pages.
  const int32_t P = c->P;
  const int32_t NB = (c->G + kDecodeCols - 1) / kDecodeCols;
  const int64_t nvs = static_cast<int64_t>(n_seqs) * c->Hkv * NB;  // (sequence, KV head, head block)
  std::vector<int32_t> &seg_lo = c->scratch_i32;  // [nvs][2]: first visible page, count
  seg_lo.assign(static_cast<size_t>(nvs) * 2, 0);
  int64_t total = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const SeqLayer &s = c->sl(layer, seq_ids[b]);
    const int32_t p = s.kv_len - 1;
    for (int32_t g = 0; g < c->Hkv; ++g) {
      const Segment &sg = c->seg(layer, seq_ids[b], g);
      const int32_t w = c->win(layer, g);
      const int32_t lo = w > 0 ? std::max(0, p - w + 1) : 0;
      const int32_t pg_lo = (lo - sg.first_token) / P;
      const int32_t pg_hi = (p - sg.first_token) / P + 1;
      for (int32_t hb = 0; hb < NB; ++hb) {
        const size_t vs = (static_cast<size_t>(b) * c->Hkv + g) * NB + hb;
        seg_lo[vs * 2] = pg_lo;
        seg_lo[vs * 2 + 1] = pg_hi - pg_lo;
        total += pg_hi - pg_lo;
      }
    }
  }
  const int64_t slots = std::max<int64_t>(1, static_cast<int64_t>(c->num_cus) * kDecodeWgPerCu);
  const int64_t n_wg = std::max<int64_t>(1, std::min(slots, ceil_div(total, c->decode_pps)));
  std::vector<DecodeItem> ditems;
  std::vector<int32_t> wg_off;
  ditems.reserve(static_cast<size_t>(n_wg + nvs));
  wg_off.reserve(static_cast<size_t>(n_wg + 1));
  std::vector<CombineItem> &citems = c->scratch_citems;
  citems.clear();
  {
    // first pass: pieces per segment and head block (for part numbering)
    const int64_t nseg = nvs;
    std::vector<int32_t> seg_parts(static_cast<size_t>(nseg), 0), seg_part0(static_cast<size_t>(nseg), 0);
    // (sequence, KV head, first query head of the block within the group) of virtual segment i
    auto vseg = [&](int64_t i, int32_t *b, int32_t *g, int32_t *head0) {
      *b = static_cast<int32_t>(i / (static_cast<int64_t>(c->Hkv) * NB));
      *g = static_cast<int32_t>((i / NB) % c->Hkv);
      *head0 = static_cast<int32_t>(i % NB) * kDecodeCols;
    };
    // Shares of equal cost: pages plus one 64-key chunk's time per piece (a
    // share's pieces each load their queries and merge their partial).
    std::vector<int32_t> lens(static_cast<size_t>(nseg));
    for (int64_t i = 0; i < nseg; ++i) lens[static_cast<size_t>(i)] = seg_lo[static_cast<size_t>(i) * 2 + 1];
    const std::vector<int64_t> bnd = decode_share_bounds(lens, total, n_wg, ceil_div(kDecodePieceCostKeys, P));
    auto share = [&](int64_t w) { return bnd[static_cast<size_t>(w)]; };
    for (int pass = 0; pass < 2; ++pass) {
      int64_t si = 0, seg_start = 0;  // current segment and its first global page index
      std::vector<int32_t> used(pass ? static_cast<size_t>(nseg) : 0, 0);
      for (int64_t w = 0; w < n_wg; ++w) {
        if (pass) wg_off.push_back(static_cast<int32_t>(ditems.size()));
        int64_t pos = share(w);
        const int64_t end = share(w + 1);
        while (pos < end) {
          while (seg_start + seg_lo[static_cast<size_t>(si) * 2 + 1] <= pos) {
            seg_start += seg_lo[static_cast<size_t>(si) * 2 + 1];
            ++si;
          }
          const int64_t seg_end = seg_start + seg_lo[static_cast<size_t>(si) * 2 + 1];
          const int64_t stop = std::min(end, seg_end);
          if (!pass) {
            seg_parts[static_cast<size_t>(si)]++;
          } else {
            int32_t b, g, head0;
            vseg(si, &b, &g, &head0);
            const int32_t pg0 = seg_lo[static_cast<size_t>(si) * 2] + static_cast<int32_t>(pos - seg_start);
            const int32_t pg1 = seg_lo[static_cast<size_t>(si) * 2] + static_cast<int32_t>(stop - seg_start);
            const int32_t part = seg_part0[static_cast<size_t>(si)] + used[static_cast<size_t>(si)]++;
            ditems.push_back(DecodeItem{b, g, pg0, pg1, part, seg_part0[static_cast<size_t>(si)],
                                        seg_parts[static_cast<size_t>(si)], head0});
          }
          pos = stop;
        }
      }
      if (!pass) {
        int32_t acc = 0;
        for (int64_t i = 0; i < nseg; ++i) {
          seg_part0[static_cast<size_t>(i)] = acc;
          acc += seg_parts[static_cast<size_t>(i)];
          if (seg_parts[static_cast<size_t>(i)] > 1) {
            int32_t b, g, head0;
            vseg(i, &b, &g, &head0);
            citems.push_back(CombineItem{seg_part0[static_cast<size_t>(i)], seg_parts[static_cast<size_t>(i)], b, 1,
                                         g * c->G + head0, std::min(kDecodeCols, c->G - head0), 0, 0});
          }
        }
        n_parts_total = acc;
      }
    }
    wg_off.push_back(static_cast<int32_t>(ditems.size()));
  }
  const int32_t n_parts = n_parts_total;

  const SeqTables tl = seq_tables_layout(c, layer, n_seqs, seq_ids);
  const size_t tbytes = align_up(tl.bytes, 16);
  const size_t ibytes = align_up(sizeof(DecodeItem) * ditems.size(), 16);
  const size_t obytes = align_up(sizeof(int32_t) * wg_off.size(), 16);
  const size_t cbytes = sizeof(CombineItem) * citems.size();
  const size_t bytes = tbytes + ibytes + obytes + cbytes;
  const size_t part_bytes = static_cast<size_t>(n_parts) * kDecodeCols * (c->D + 1) * sizeof(float);
  float *parts = nullptr;
  rc = carve(c, base, cap, bytes, part_bytes, &parts);
  if (rc) return rc;
  if (no_alloc && bytes > c->h_stage_cap[c->stage_next])
    return c->fail(SEGKV_E_NOMEM, "decode tables of %zu bytes exceed the host staging buffer of %zu bytes", bytes,
                   c->h_stage_cap[c->stage_next]);
  char *stage = nullptr;
  int slot = 0;
  rc = acquire_stage(c, bytes, &stage, &slot);
  if (rc) return rc;
  write_seq_tables(c, layer, n_seqs, seq_ids, nullptr, nullptr, tl, stage);
  std::memcpy(stage + tbytes, ditems.data(), sizeof(DecodeItem) * ditems.size());
  std::memcpy(stage + tbytes + ibytes, wg_off.data(), sizeof(int32_t) * wg_off.size());
  if (cbytes) std::memcpy(stage + tbytes + ibytes + obytes, citems.data(), cbytes);
  rc = upload(c, slot, bytes, base);
  if (rc) return rc;

  DecodeArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.k_pool = c->k_pool;
  a.v_pool = c->v_pool;
  a.seqs = reinterpret_cast<const SeqDesc *>(base);
  a.segs = reinterpret_cast<const SegDesc *>(base + tl.seg_off);
  a.page_ids = reinterpret_cast<const int32_t *>(base + tl.pid_off);
  a.rope = rope_args(c, tl, base);
  a.items = reinterpret_cast<const DecodeItem *>(base + tbytes);
  a.wg_piece_off = reinterpret_cast<const int32_t *>(base + tbytes + ibytes);
  a.part_o = parts;
  a.part_lse = parts ? parts + static_cast<size_t>(n_parts) * kDecodeCols * c->D : nullptr;
  a.o = static_cast<uint16_t *>(o);
  a.lse = lse;
  a.num_q_heads = c->Hq;
  a.num_kv_heads = c->Hkv;
  a.group = c->G;
  a.scale = c->scale;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  TimedLaunch t{};
  rc = timed_begin(c, &t, SEGKV_KERNEL_DECODE_SPLIT);
  if (rc) return rc;
  hipError_t e = launch_decode(a, static_cast<int>(n_wg), c->D, c->P, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "decode launch");
  rc = timed_end(c, &t);
  if (rc || citems.empty()) return rc;
  CombineArgs ca;
  ca.part_o = a.part_o;
  ca.part_lse = a.part_lse;
  ca.items = reinterpret_cast<const CombineItem *>(base + tbytes + ibytes + obytes);
  ca.o = static_cast<uint16_t *>(o);
  ca.lse = lse;
  ca.num_q_heads = c->Hq;
  ca.slot_rows = kDecodeCols;
  TimedLaunch t2{};
  rc = timed_begin(c, &t2, SEGKV_KERNEL_COMBINE);
  if (rc) return rc;
  e = launch_combine(ca, static_cast<int>(citems.size()), std::min(kDecodeCols, c->G), c->D, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "combine launch");
  return timed_end(c, &t2);
}

}  // namespace

extern "C" {

int segkv_decode(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const void *q, void *o,
                 float *lse) {
  if (!c) return SEGKV_E_INVAL;
  return decode_impl(c, layer, n_seqs, seq_ids, q, o, lse, c->ws, c->ws_bytes, false);
}

int segkv_decode_noalloc(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const void *q,
                         void *o, float *lse) {
  if (!c) return SEGKV_E_INVAL;
  if (c->planning) return c->fail(SEGKV_E_STATE, "decode needs device pools (planning-only context)");
  // No timing events (creating one allocates); the mask is left as it is.
  const int32_t mask = c->timing_mask;
  c->timing_mask = 0;
  const int rc = decode_impl(c, layer, n_seqs, seq_ids, q, o, lse, c->fixed_scratch, kStaticScratchBytes, true);
  c->timing_mask = mask;
  return rc;
}

int segkv_token_scores(segkv_ctx *c, int32_t layer, int32_t n_seqs, const int32_t *seq_ids, const int32_t *cu_q,
                       const void *q, const float *lse, float *scores) {
  if (!c) return SEGKV_E_INVAL;
  if (c->planning) return c->fail(SEGKV_E_STATE, "token scores need device pools (planning-only context)");
  int rc = check_layer_seqs(c, layer, n_seqs, seq_ids);
  if (rc) return rc;
  if (n_seqs == 0) return SEGKV_OK;
  if (!cu_q) return c->fail(SEGKV_E_INVAL, "cu_q is NULL");
  if (cu_q[0] != 0) return c->fail(SEGKV_E_INVAL, "cu_q[0] must be 0");
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int32_t ql = cu_q[b + 1] - cu_q[b];
    const SeqLayer &s = c->sl(layer, seq_ids[b]);
    if (ql < 0) return c->fail(SEGKV_E_INVAL, "cu_q must be non-decreasing");
    if (ql > s.kv_len) return c->fail(SEGKV_E_INVAL, "q_len %d > kv_len %d (seq %d)", ql, s.kv_len, seq_ids[b]);
    if (ql > 0 && s.kv_len - ql < s.pending_from)
      return c->fail(SEGKV_E_INVAL, "seq %d: queries start before the earliest pending query", seq_ids[b]);
    for (int32_t b2 = 0; b2 < b; ++b2)
      if (seq_ids[b2] == seq_ids[b]) return c->fail(SEGKV_E_INVAL, "duplicate seq id %d", seq_ids[b]);
  }
  if (cu_q[n_seqs] == 0) return SEGKV_OK;
  if (!q || !lse || !scores) return c->fail(SEGKV_E_INVAL, "q / lse / scores is NULL");

  // Items over the chunk's tiles only, in canonical order (sequence, KV
  // head, q tile, tile range); long items are cut like the prefill's.
  const int32_t G = c->G;
  const int32_t rows = kPrefillRows / G;
  std::vector<PrefillItem> items;
  int64_t total_cost = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    const int32_t ql = cu_q[b + 1] - cu_q[b];
    const SeqLayer &s = c->sl(layer, seq_ids[b]);
    const int32_t base = s.kv_len - ql;
    for (int32_t g = 0; g < c->Hkv; ++g) {
      const int32_t w = c->win(layer, g);
      for (int32_t qt = 0; qt * rows < ql; ++qt) {
        const int32_t p_min = base + qt * rows;
        const int32_t p_max = base + std::min((qt + 1) * rows, ql) - 1;
        const int32_t lo = w > 0 ? std::max(0, p_min - w + 1) : 0;
        const int32_t tb = std::max(lo, base) / kTileKeys;
        const int32_t te = p_max / kTileKeys + 1;
        items.push_back(PrefillItem{b, g, qt, tb, te, 0, 0, 0});
        total_cost += te - tb;
      }
    }
  }
  // Pieces of at most `split` tiles; a persistent grid of resident
  // workgroups takes them from a queue, longest first (sorted below), so
  // workgroups that run faster (the CU's arbitration favours older waves)
  // take more of them.
  int64_t split = c->prefill_split_tiles;
  if (split <= 0) {
    const int64_t slots = std::max<int64_t>(1, static_cast<int64_t>(c->num_cus) * kScoreWgPerCu);
    split = std::max<int64_t>(kMinSplitTiles, ceil_div(total_cost, kScorePiecesPerSlot * slots));
  }
  std::vector<PrefillItem> cut;
  int32_t n_part_rows = 0;
  for (const PrefillItem &x : items) {
    const int32_t per = static_cast<int32_t>(std::min<int64_t>(split, std::max(1, x.tile_end - x.tile_begin)));
    for (int32_t t0 = x.tile_begin; t0 < x.tile_end; t0 += per) {
      const int32_t t1 = std::min(x.tile_end, t0 + per);
      cut.push_back(PrefillItem{x.seq, x.kv_head, x.qtile, t0, t1, n_part_rows, 0, 0});
      n_part_rows += t1 - t0;
    }
  }
  // Reduction lists: per (sequence, chunk tile), the partial rows covering
  // it in canonical item order.
  std::vector<ScoreRow> srows;
  std::vector<int32_t> pidx;
  {
    size_t first = 0;
    for (int32_t b = 0; b < n_seqs; ++b) {
      const int32_t ql = cu_q[b + 1] - cu_q[b];
      size_t last = first;
      while (last < cut.size() && cut[last].seq == b) ++last;
      if (ql > 0) {
        const SeqLayer &s = c->sl(layer, seq_ids[b]);
        const int32_t ct0 = (s.kv_len - ql) / kTileKeys, ct1 = (s.kv_len - 1) / kTileKeys + 1;
        for (int32_t t = ct0; t < ct1; ++t) {
          ScoreRow r{b, t, static_cast<int32_t>(pidx.size()), 0};
          for (size_t i = first; i < last; ++i)
            if (cut[i].tile_begin <= t && t < cut[i].tile_end) pidx.push_back(cut[i].part + (t - cut[i].tile_begin));
          r.end = static_cast<int32_t>(pidx.size());
          srows.push_back(r);
        }
      }
      first = last;
    }
  }
  // Longest first (the sums do not depend on the order).
  std::stable_sort(cut.begin(), cut.end(), [](const PrefillItem &x, const PrefillItem &y) {
    return x.tile_end - x.tile_begin > y.tile_end - y.tile_begin;
  });
  const int64_t n_wgs = std::min<int64_t>(static_cast<int64_t>(cut.size()),
                                          std::max<int64_t>(1, static_cast<int64_t>(c->num_cus) * kScoreWgPerCu));

  const SeqTables tl = seq_tables_layout(c, layer, n_seqs, seq_ids);
  const size_t tbytes = align_up(tl.bytes, 16);
  const size_t ibytes = align_up(sizeof(PrefillItem) * cut.size(), 16);
  const size_t rbytes = align_up(sizeof(ScoreRow) * srows.size(), 16);
  const size_t pbytes = align_up(sizeof(int32_t) * pidx.size(), 16);
  const size_t bytes = tbytes + ibytes + rbytes + pbytes + 16;  // + the queue counter (uploaded as 0)
  float *parts = nullptr;
  rc = carve(c, c->ws, c->ws_bytes, bytes, static_cast<size_t>(std::max(n_part_rows, 1)) * kTileKeys * sizeof(float),
             &parts);
  if (rc) return rc;
  char *stage = nullptr;
  int slot = 0;
  rc = acquire_stage(c, bytes, &stage, &slot);
  if (rc) return rc;
  std::vector<int32_t> qs(n_seqs), qlv(n_seqs);
  for (int32_t b = 0; b < n_seqs; ++b) {
    qs[b] = cu_q[b];
    qlv[b] = cu_q[b + 1] - cu_q[b];
  }
  write_seq_tables(c, layer, n_seqs, seq_ids, qs.data(), qlv.data(), tl, stage);
  std::memcpy(stage + tbytes, cut.data(), sizeof(PrefillItem) * cut.size());
  std::memcpy(stage + tbytes + ibytes, srows.data(), sizeof(ScoreRow) * srows.size());
  if (!pidx.empty()) std::memcpy(stage + tbytes + ibytes + rbytes, pidx.data(), sizeof(int32_t) * pidx.size());
  std::memset(stage + tbytes + ibytes + rbytes + pbytes, 0, 16);
  rc = upload(c, slot, bytes, c->ws);
  if (rc) return rc;

  ScoreArgs a;
  a.q = static_cast<const uint16_t *>(q);
  a.lse = lse;
  a.k_pool = c->k_pool;
  a.seqs = reinterpret_cast<const SeqDesc *>(c->ws);
  a.segs = reinterpret_cast<const SegDesc *>(c->ws + tl.seg_off);
  a.page_ids = reinterpret_cast<const int32_t *>(c->ws + tl.pid_off);
  a.rope = rope_args(c, tl, c->ws);
  a.items = reinterpret_cast<const PrefillItem *>(c->ws + tbytes);
  a.counter = reinterpret_cast<int32_t *>(c->ws + tbytes + ibytes + rbytes + pbytes);
  a.n_items = static_cast<int32_t>(cut.size());
  a.part = parts;
  a.num_q_heads = c->Hq;
  a.num_kv_heads = c->Hkv;
  a.group = G;
  a.rows_per_tile = rows;
  a.scale_log2 = c->scale * 1.4426950408889634f;
  TimedLaunch t{};
  rc = timed_begin(c, &t, SEGKV_KERNEL_SCORE);
  if (rc) return rc;
  hipError_t e = launch_score(a, static_cast<int>(n_wgs), c->D, c->P, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "score launch");
  rc = timed_end(c, &t);
  if (rc) return rc;
  ScoreReduceArgs ra;
  ra.part = parts;
  ra.part_idx = reinterpret_cast<const int32_t *>(c->ws + tbytes + ibytes + rbytes);
  ra.rows = reinterpret_cast<const ScoreRow *>(c->ws + tbytes + ibytes);
  ra.seqs = a.seqs;
  ra.scores = scores;
  ra.n_rows = static_cast<int32_t>(srows.size());
  TimedLaunch t2{};
  rc = timed_begin(c, &t2, SEGKV_KERNEL_SCORE_REDUCE);
  if (rc) return rc;
  e = launch_score_reduce(ra, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "score reduce launch");
  return timed_end(c, &t2);
}

int segkv_topk(segkv_ctx *c, int32_t n_seqs, const int32_t *cu_n, const float *scores, const int32_t *k,
               int32_t *out_idx) {
  if (!c) return SEGKV_E_INVAL;
  if (c->planning) return c->fail(SEGKV_E_STATE, "top-k needs a device context (planning-only context)");
  if (n_seqs < 0) return c->fail(SEGKV_E_INVAL, "n_seqs < 0");
  if (n_seqs == 0) return SEGKV_OK;
  if (!cu_n || !k) return c->fail(SEGKV_E_INVAL, "cu_n / k is NULL");
  if (cu_n[0] != 0) return c->fail(SEGKV_E_INVAL, "cu_n[0] must be 0");
  int64_t total_k = 0;
  for (int32_t b = 0; b < n_seqs; ++b) {
    if (cu_n[b + 1] < cu_n[b]) return c->fail(SEGKV_E_INVAL, "cu_n must be non-decreasing");
    if (k[b] < 0 || k[b] > cu_n[b + 1] - cu_n[b])
      return c->fail(SEGKV_E_INVAL, "k[%d] = %d must be in [0, %d]", b, k[b], cu_n[b + 1] - cu_n[b]);
    total_k += k[b];
  }
  if (total_k == 0) return SEGKV_OK;
  if (!scores || !out_idx) return c->fail(SEGKV_E_INVAL, "scores / out_idx is NULL");
  const size_t nb = static_cast<size_t>(n_seqs);
  const size_t cu_bytes = align_up(sizeof(int32_t) * (nb + 1), 16);
  const size_t k_bytes = align_up(sizeof(int32_t) * nb, 16);
  const size_t bytes = cu_bytes + 2 * k_bytes;
  float *unused = nullptr;
  int rc = carve(c, c->ws, c->ws_bytes, bytes, 0, &unused);
  if (rc) return rc;
  char *stage = nullptr;
  int slot = 0;
  rc = acquire_stage(c, bytes, &stage, &slot);
  if (rc) return rc;
  std::memcpy(stage, cu_n, sizeof(int32_t) * (nb + 1));
  std::memcpy(stage + cu_bytes, k, sizeof(int32_t) * nb);
  int32_t *off = reinterpret_cast<int32_t *>(stage + cu_bytes + k_bytes);
  int32_t acc = 0;
  for (size_t b = 0; b < nb; ++b) {
    off[b] = acc;
    acc += k[b];
  }
  rc = upload(c, slot, bytes, c->ws);
  if (rc) return rc;
  TopkArgs a;
  a.scores = scores;
  a.cu = reinterpret_cast<const int32_t *>(c->ws);
  a.k = reinterpret_cast<const int32_t *>(c->ws + cu_bytes);
  a.out_off = reinterpret_cast<const int32_t *>(c->ws + cu_bytes + k_bytes);
  a.out = out_idx;
  TimedLaunch t{};
  rc = timed_begin(c, &t, SEGKV_KERNEL_TOPK);
  if (rc) return rc;
  hipError_t e = launch_topk(a, n_seqs, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "top-k launch");
  return timed_end(c, &t);
}

int segkv_merge(segkv_ctx *c, int64_t n_rows, const void *o_a, const float *lse_a, const void *o_b,
                const float *lse_b, const uint8_t *mode, void *o, float *lse) {
  if (!c) return SEGKV_E_INVAL;
  if (c->planning) return c->fail(SEGKV_E_STATE, "merge needs a device context (planning-only context)");
  if (n_rows < 0) return c->fail(SEGKV_E_INVAL, "n_rows < 0");
  if (n_rows == 0) return SEGKV_OK;
  if (n_rows > std::numeric_limits<int64_t>::max() / (static_cast<int64_t>(c->Hq) * c->D * 2))
    return c->fail(SEGKV_E_INVAL, "n_rows too large");
  if (!o_a || !lse_a || !o_b || !lse_b || !mode || !o)
    return c->fail(SEGKV_E_INVAL, "o_a, lse_a, o_b, lse_b, mode and o must be set");
  auto misaligned = [](const void *p, uintptr_t a) { return reinterpret_cast<uintptr_t>(p) % a != 0; };
  if (misaligned(o_a, 16) || misaligned(o_b, 16) || misaligned(o, 16))
    return c->fail(SEGKV_E_INVAL, "o_a, o_b and o must be 16-byte aligned");
  if (misaligned(lse_a, 4) || misaligned(lse_b, 4) || (lse && misaligned(lse, 4)))
    return c->fail(SEGKV_E_INVAL, "lse arrays must be 4-byte aligned");
  MergeArgs a;
  a.o_a = static_cast<const uint16_t *>(o_a);
  a.lse_a = lse_a;
  a.o_b = static_cast<const uint16_t *>(o_b);
  a.lse_b = lse_b;
  a.mode = mode;
  a.o = static_cast<uint16_t *>(o);
  a.lse = lse;
  a.n_pairs = n_rows * c->Hq;
  const int64_t per_wg = static_cast<int64_t>(kMergeThreads / (c->D / 8)) * kMergeUnroll;
  const int64_t n_wgs = std::min<int64_t>(ceil_div(a.n_pairs, per_wg), static_cast<int64_t>(c->num_cus) * 8);
  TimedLaunch t{};
  int rc = timed_begin(c, &t, SEGKV_KERNEL_MERGE);
  if (rc) return rc;
  hipError_t e = launch_merge(a, static_cast<int>(n_wgs), c->D, c->stream);
  if (e != hipSuccess) return c->device_fail(e, "merge launch");
  return timed_end(c, &t);
}

int segkv_set_timing(segkv_ctx *c, int32_t kernel_mask) {
  if (!c) return SEGKV_E_INVAL;
  if (c->planning) return c->fail(SEGKV_E_STATE, "timing needs a device context");
  if (kernel_mask & ~((1 << SEGKV_KERNEL_COUNT) - 1))
    return c->fail(SEGKV_E_INVAL, "timing mask 0x%x names unknown kernels", kernel_mask);
  int rc = drain_timing(c);
  if (rc) return rc;
  for (int k = 0; k < SEGKV_KERNEL_COUNT; ++k) {
    c->tot_ms[k] = 0.0;
    c->launches[k] = 0;
  }
  c->timing_mask = kernel_mask;
  return SEGKV_OK;
}

int segkv_read_timing(segkv_ctx *c, int32_t kernel, double *total_ms, int64_t *launches) {
  if (!c) return SEGKV_E_INVAL;
  if (kernel < 0 || kernel >= SEGKV_KERNEL_COUNT) return c->fail(SEGKV_E_INVAL, "unknown kernel id %d", kernel);
  int rc = drain_timing(c);
  if (rc) return rc;
  if (total_ms) *total_ms = c->tot_ms[kernel];
  if (launches) *launches = c->launches[kernel];
  return SEGKV_OK;
}

int segkv_set_tuning(segkv_ctx *c, int32_t knob, int64_t value) {
  if (!c) return SEGKV_E_INVAL;
  switch (knob) {
    case SEGKV_TUNE_DECODE_MIN_PAGES:
      if (value > (1 << 20)) return c->fail(SEGKV_E_INVAL, "pages per split too large");
      c->decode_pps = value > 0 ? static_cast<int32_t>(value) : kDefaultDecodeMinPages;
      return SEGKV_OK;
    case SEGKV_TUNE_PREFILL_SPLIT_TILES:
      c->prefill_split_tiles = value > 0 ? value : kDefaultPrefillSplitTiles;
      return SEGKV_OK;
    case SEGKV_TUNE_PREFILL_ORDER:
      if (value > 1) return c->fail(SEGKV_E_INVAL, "prefill order must be 0 (longest first) or 1 (XCD-aware)");
      c->prefill_order = value > 0 ? static_cast<int32_t>(value) : 0;
      return SEGKV_OK;
    case SEGKV_TUNE_PREFILL_KERNEL:
      if (value > kPrefillDuo)
        return c->fail(SEGKV_E_INVAL, "prefill kernel must be 0 (default), 1 (8 x 32 rows), 2 (4 x 64 rows), "
                                      "3 (two groups), 4 (pipelined) or 5 (two workgroups per CU)");
      if (value == kPrefillDuo && c->G > kPrefillDuoRows)
        return c->fail(SEGKV_E_INVAL, "prefill kernel 5 needs num_q_heads / num_kv_heads <= %d", kPrefillDuoRows);
      c->prefill_kernel = value > 0 ? static_cast<int32_t>(value) : 0;
      return SEGKV_OK;
    default:
      return c->fail(SEGKV_E_INVAL, "unknown tuning knob %d", knob);
  }
}

}  // extern "C"
