// Host-side launchers of the compressor kernels (enqueue only).
#pragma once

#include <hip/hip_runtime.h>

#include "kernel_args.h"

namespace ds4c {

hipError_t launch_proj(const ProjArgs& a, int in_dtype, hipStream_t stream);
// Ratio-4 layers pool in one launch, ratio-128 layers in two (phase 0: partial
// pools, phase 1: merge, finish and frontier carry).
int pool_launches(int ratio);
hipError_t launch_pool(const PoolArgs& a, int phase, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int in_dtype, hipStream_t stream);
hipError_t launch_fill(const FillArgs& f, hipStream_t stream);

}  // namespace ds4c
