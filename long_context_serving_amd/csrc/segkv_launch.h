// Kernel launchers of libsegkv (host side).  The argument structures and
// constants they take are in segkv_internal.h.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "segkv_internal.h"

namespace segkv {

// Timing events for the next launch on the calling thread.  When the host
// times a kernel it sets them; the launch hands them to the dispatch itself
// (hipExtLaunchKernelGGL), which stamps the kernel's own start and end, so
// the elapsed time is the kernel's execution without the cost of separate
// event-record commands.  `used` tells the host that a launch took them.
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
  bool used = false;
};
LaunchEvents &launch_events();

// Every kernel of the library is launched through this.
#define SEGKV_LAUNCH(KERNEL, GRID, BLOCK, STREAM, ...)                                                  \
  do {                                                                                                 \
    ::segkv::LaunchEvents &ev_ = ::segkv::launch_events();                                             \
    ev_.used = ev_.start != nullptr;                                                                   \
    hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, 0, STREAM, ev_.start, ev_.stop, 0, __VA_ARGS__);        \
  } while (0)

// Shape of the two-workgroup prefill variant (prefill_variants.hip): 4 waves
// of 32 rows per workgroup, 128 rows per work item, two workgroups per CU.
constexpr int kPrefillDuoThreads = 256;
constexpr int kPrefillDuoRows = 128;
constexpr int kPrefillDuoWgPerCu = 2;

// Launchers (csrc/*.hip, one file per kernel family).  Return the launch status.
hipError_t launch_scatter(const ScatterArgs &a, int n_items, int head_dim, int page_size, hipStream_t s);
hipError_t launch_prefill(const PrefillArgs &a, int n_items, int head_dim, int page_size, hipStream_t s);
hipError_t launch_prefill_sp(const PrefillArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s);
hipError_t launch_prefill_pp(const PrefillArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s);
hipError_t launch_prefill_wide(const PrefillArgs &a, int n_items, int head_dim, int page_size, hipStream_t s);
hipError_t launch_prefill_duo(const PrefillArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s);
hipError_t launch_decode(const DecodeArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s);
hipError_t launch_combine(const CombineArgs &a, int n_items, int max_entries, int head_dim, hipStream_t s);
hipError_t launch_merge(const MergeArgs &a, int n_wgs, int head_dim, hipStream_t s);
hipError_t launch_score(const ScoreArgs &a, int n_wgs, int head_dim, int page_size, hipStream_t s);
hipError_t launch_score_reduce(const ScoreReduceArgs &a, hipStream_t s);
hipError_t launch_topk(const TopkArgs &a, int n_seqs, hipStream_t s);
// bytes are rounded up to 16; both buffers must hold the rounded size
hipError_t launch_upload(void *dst, const void *src_pinned, size_t bytes, hipStream_t s);

// The address of the fixed device scratch of segkv_decode_noalloc (decode.hip)
// on the current device (resolved once per device).
hipError_t scratch_address(void **out);

}  // namespace segkv
