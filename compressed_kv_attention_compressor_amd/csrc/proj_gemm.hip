// Projection GEMM: out[t, c] = sum_h x[t, h] * W_seg[c - col0, h] for the
// four weight blocks of a layer (wkv and wgate of each lane, Part 3 §4),
// written as one [T, N] float32 matrix.  Both operands are K-contiguous.
//
// First version: a plain LDS-tiled float FMA kernel, 64 x 64 tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_args.h"
#include "launch.h"

namespace ds4c {

namespace {

constexpr int kTile = 64;
constexpr int kKStep = 16;

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

template <typename Tin>
__global__ void __launch_bounds__(256) proj_gemm_kernel(ProjArgs a) {
  __shared__ float As[kKStep][kTile + 1];
  __shared__ float Bs[kKStep][kTile + 1];
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && blockIdx.y == 0)
    for (int i = tid; i < a.n_zero; i += blockDim.x) a.zero_ptr[i] = 0u;

  const int col0 = blockIdx.x * kTile;
  const int64_t row0 = (int64_t)blockIdx.y * kTile;
  int s = 0;
  while (s + 1 < a.n_seg && col0 >= a.seg[s + 1].col0) ++s;
  const Tin* B = reinterpret_cast<const Tin*>(a.seg[s].w) + (int64_t)(col0 - a.seg[s].col0) * a.K;
  const Tin* A = reinterpret_cast<const Tin*>(a.x);

  const int tx = tid % 16, ty = tid / 16;
  float acc[4][4] = {};
  const int lr = tid / 4, lk = (tid % 4) * 4;
  for (int k0 = 0; k0 < a.K; k0 += kKStep) {
    const int64_t ar = row0 + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      As[lk + i][lr] = ar < a.M ? to_f32(A[ar * a.K + k0 + lk + i]) : 0.f;
      Bs[lk + i][lr] = to_f32(B[(int64_t)lr * a.K + k0 + lk + i]);
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kKStep; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        av[i] = As[kk][ty * 4 + i];
        bv[i] = Bs[kk][tx * 4 + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t r = row0 + ty * 4 + i;
    if (r < a.M) {
#pragma unroll
      for (int j = 0; j < 4; ++j) a.out[r * a.N + col0 + tx * 4 + j] = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_proj(const ProjArgs& a, int in_dtype, hipStream_t stream) {
  dim3 grid((unsigned)(a.N / kTile), (unsigned)((a.M + kTile - 1) / kTile));
  if (in_dtype == 1)
    hipLaunchKernelGGL(proj_gemm_kernel<uint16_t>, grid, dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL(proj_gemm_kernel<float>, grid, dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace ds4c
