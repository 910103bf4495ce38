// Kernel launchers of libsegkv (host side).  The argument structures and
// constants they take are in segkv_internal.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "segkv_internal.h"

namespace segkv {

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
