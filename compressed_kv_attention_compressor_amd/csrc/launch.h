// Host-side launchers of the compressor kernels (enqueue only).
#pragma once

#include <hip/hip_runtime_api.h>

#include "kernel_args.h"

namespace ds4c {

// Events the dispatch itself records around a kernel (AMD's extended
// launch), so a timed kernel's interval excludes host launch overhead.  Both
// null when not timing; a multi-launch step gives start to its first kernel
// and stop to its last.
struct Timing {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

// Plain (unfused) projection: tile rows (256, 128 or 64) and the number of K
// ranges, chosen by estimated time.  A call with few output tiles splits K
// so that more workgroups run; split s writes plane s of the output and a
// second launch adds the planes into plane 0 in order.  A split keeps
// k_split * M <= kSplitRows, so the planes of a call with M tokens take at
// most max(M, min(kSplitRows, 16 M)) rows of N floats.
constexpr int64_t kSplitRows = 1024;
struct ProjPlan {
  int bm;
  int k_split;
};
ProjPlan proj_plan(int64_t M, int N, int K);
// Whether a call that starts on a window boundary pools inside the
// projection epilogue (M tokens, N projection columns, K = hidden, d_tot =
// pooled dims of all lanes): yes unless the fused grid is so small that the
// plain path is faster (measured), which happens for short calls.  Calls
// with small hidden sizes always take the fused path.
bool use_fused_projection(int ratio, int64_t M, int N, int K, int d_tot);

hipError_t launch_proj(const ProjArgs& a, int in_dtype, hipStream_t stream, const Timing& tm);
// Ratio-4 layers and fused calls pool in one launch; plain ratio-128 calls in
// two (phase 0: partial pools, phase 1: merge, finish and frontier carry).
int pool_launches(const PoolArgs& a);
hipError_t launch_pool(const PoolArgs& a, int phase, hipStream_t stream, const Timing& tm);
// The GEMV launch is timed by `tm`, the window-boundary launches (if any) by `tm_pool`.
hipError_t launch_decode(const DecodeArgs& a, int in_dtype, hipStream_t stream, const Timing& tm,
                         const Timing& tm_pool);
hipError_t launch_fill(const FillArgs& f, hipStream_t stream, const Timing& tm);
// Reads or writes `bytes` (a multiple of 16) of a 16-byte aligned device buffer.
hipError_t launch_evict(void* p, size_t bytes, bool write, hipStream_t stream);
// Indexer: scores per row, then a radix top-k.  One select workgroup takes
// up to kIndexerChunk rows; longer calls select per chunk first, and the
// final pass takes at most kIndexerMaxCand surviving keys (n_chunks * k).
constexpr int kIndexerChunk = 32768;
constexpr int kIndexerMaxCand = 16384;
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream, const Timing& tm);
// Allocation-free indexer calls use a fixed device array of this many bytes
// (the workspace of a call of 1,048,576 rows at k = 512, the largest of any
// call up to that many rows); indexer_scratch returns the current device's
// copy (looked up once per device).
constexpr size_t kIndexerScratchBytes = 8519936;
hipError_t indexer_scratch(void** ptr);
// Mixed attention: a partial launch over (item chunks of 32, head groups of
// 8), then a merge launch per head.
int mixed_attn_splits(int n_items);
hipError_t launch_mixed_attention(const MixedAttnArgs& a, hipStream_t stream, const Timing& tm);

}  // namespace ds4c
