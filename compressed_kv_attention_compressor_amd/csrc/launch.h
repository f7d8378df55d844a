// Host-side launchers of the compressor kernels (enqueue only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

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

hipError_t launch_proj(const ProjArgs& a, int in_dtype, hipStream_t stream, const Timing& tm);
// Ratio-4 layers and fused calls pool in one launch; plain ratio-128 calls in
// two (phase 0: partial pools, phase 1: merge, finish and frontier carry).
int pool_launches(const PoolArgs& a);
hipError_t launch_pool(const PoolArgs& a, int phase, hipStream_t stream, const Timing& tm);
hipError_t launch_decode(const DecodeArgs& a, int in_dtype, hipStream_t stream, const Timing& tm);
hipError_t launch_fill(const FillArgs& f, hipStream_t stream, const Timing& tm);

}  // namespace ds4c
