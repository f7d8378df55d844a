// Fused compressor pool kernels: APE add, window gather (projection
// workspace or carried frontier), per-dimension softmax pool, RMS norm, tail
// RoPE, FP8 / Hadamard+FP4 round trip, row append and frontier carry, in one
// launch per prefill call.
//
// What is pooled (Part 3 §4, §5): for every output dim j, the window's
// entries (kv, score + APE[pos % ratio]) are weighted by exp(score - max)
// and averaged.  A ratio-128 row pools tokens 128k .. 128k+127 on columns
// [0, D).  A ratio-4 row pools tokens 4k-4 .. 4k-1 on columns [0, D) (the
// previous half of the 8-row frontier) and tokens 4k .. 4k+3 on columns
// [D, 2D) (the current half); tokens before position 0 are empty.
//
// Tokens before the call (positions < n0) are read from the frontier: for
// ratio 4 a token p lives in row 4 + p%4 when p >= n0 - n0%4, else in row
// p%4 (it was moved there by the half shift); for ratio 128 in row p%128.
// Only the first one or two windows of a call can touch such tokens; they
// are handled by the workgroup that also rewrites the frontier, after it
// has finished reading it.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace ds4c {

namespace {

constexpr int kPoolThreads = 256;

// Entries of one lane's column block for token p, DPL dims starting at
// column c of the lane's W-wide kv / score blocks.
template <int R, int DPL>
__device__ __forceinline__ void fetch_token(const PoolArgs& a, const LaneDev& L, int64_t p, int c,
                                            float (&kv)[DPL], float (&sc)[DPL]) {
  if (p < 0) {
#pragma unroll
    for (int i = 0; i < DPL; ++i) { kv[i] = 0.f; sc[i] = -INFINITY; }
    return;
  }
  const int pr = (int)(p & (R - 1));
  if (p < a.n0) {
    int row = pr;
    if (R == 4 && p >= a.n0 - (a.n0 & 3)) row = 4 + pr;
    load_vec<DPL>(kv, L.fr_kv + (int64_t)row * L.W + c);
    load_vec<DPL>(sc, L.fr_sc + (int64_t)row * L.W + c);
    return;
  }
  const float* src = a.proj + (p - a.n0) * a.ld;
  load_vec<DPL>(kv, src + L.kv_col + c);
  load_vec<DPL>(sc, src + L.sc_col + c);
  float ape[DPL];
  load_vec<DPL>(ape, L.ape + pr * L.W + c);
#pragma unroll
  for (int i = 0; i < DPL; ++i) sc[i] += ape[i];
}

// One ratio-4 row of one lane on one wave.
template <int DPL>
__device__ void r4_row(const PoolArgs& a, const LaneDev& L, int64_t k, int lane) {
  float kv[8][DPL], sc[8][DPL];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = (e < 4 ? 0 : L.D) + lane * DPL;
    fetch_token<4, DPL>(a, L, 4 * k - 4 + e, c, kv[e], sc[e]);
  }
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    float m = sc[0][i];
#pragma unroll
    for (int e = 1; e < 8; ++e) m = fmaxf(m, sc[e][i]);
    float den = 0.f, num = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = expf(sc[e][i] - m);
        den += w;
        num = fmaf(w, kv[e][i], num);
      }
    }
    o[i] = den > 0.f ? num / den : 0.f;
  }
  float* pre = L.prequant ? L.prequant + (k - a.k_lo) * L.D : nullptr;
  finish_row_wave<DPL>(o, L, a.n_rot, a.log2_base, a.rms_eps, k, 4, pre, L.rows + k * L.D, lane);
}

// Frontier carry after a call, by one whole workgroup, for both ratios.
// With n = n0 + T, c = n % ratio, m = n - c: ratio 4 keeps tokens m-4 .. m-1
// in rows 0..3 and m .. n-1 in rows 4 .. 3+c; ratio 128 keeps m .. n-1 in
// rows 0 .. c-1.  Only rows that change are written.  Every read of the
// incoming frontier by this call's windows has completed before this runs.
template <int R>
__device__ void carry_frontier(const PoolArgs& a) {
  const int64_t n = a.n0 + a.T;
  const int64_t m = n - (n & (R - 1));
  const int c4 = threadIdx.x * 4;
  if (R == 4) {
    const int64_t m0 = a.n0 - (a.n0 & 3);
    // Old tokens that move from the current half to the previous half.
    if (m > m0 && m - 4 < a.n0) {
      for (int l = 0; l < a.n_lanes; ++l) {
        const LaneDev& L = a.lane[l];
        for (int64_t p = m - 4; p < a.n0; ++p) {
          const int src = 4 + (int)(p & 3), dst = (int)(p & 3);
          for (int c = c4; c < L.W; c += 4 * kPoolThreads) {
            const float4 kv = *reinterpret_cast<const float4*>(L.fr_kv + src * L.W + c);
            const float4 sc = *reinterpret_cast<const float4*>(L.fr_sc + src * L.W + c);
            *reinterpret_cast<float4*>(L.fr_kv + dst * L.W + c) = kv;
            *reinterpret_cast<float4*>(L.fr_sc + dst * L.W + c) = sc;
          }
        }
      }
      __syncthreads();
    }
  }
  // New tokens from the projection workspace.
  const int64_t first = R == 4 ? (m - 4 > a.n0 ? m - 4 : a.n0) : (m > a.n0 ? m : a.n0);
  for (int l = 0; l < a.n_lanes; ++l) {
    const LaneDev& L = a.lane[l];
    for (int64_t p = first; p < n; ++p) {
      const int pr = (int)(p & (R - 1));
      const int row = R == 4 ? (p >= m ? 4 + pr : pr) : (int)(p - m);
      const float* src = a.proj + (p - a.n0) * a.ld;
      for (int c = c4; c < L.W; c += 4 * kPoolThreads) {
        const float4 kv = *reinterpret_cast<const float4*>(src + L.kv_col + c);
        float4 sc = *reinterpret_cast<const float4*>(src + L.sc_col + c);
        const float4 ap = *reinterpret_cast<const float4*>(L.ape + pr * L.W + c);
        sc.x += ap.x; sc.y += ap.y; sc.z += ap.z; sc.w += ap.w;
        *reinterpret_cast<float4*>(L.fr_kv + row * L.W + c) = kv;
        *reinterpret_cast<float4*>(L.fr_sc + row * L.W + c) = sc;
      }
    }
  }
}

// Ratio 4.  Workgroup 0 pools the n_head leading windows (one wave per
// (window, lane), at most 2 x 2) and then carries the frontier; every other
// workgroup pools four (window, lane) rows, one per wave.
template <int DPLA, int DPLI>
__global__ void __launch_bounds__(kPoolThreads) pool_r4_kernel(PoolArgs a) {
  const int wave = threadIdx.x / kWave;
  const int lane = threadIdx.x % kWave;
  // Jobs are (window, lane) pairs, lane = job & 1 (ratio-4 layers have two).
  int64_t job;
  if (blockIdx.x == 0) {
    job = wave < 2 * a.n_head ? wave : -1;
  } else {
    job = 2 * a.n_head + (int64_t)(blockIdx.x - 1) * (kPoolThreads / kWave) + wave;
  }
  if (job >= 0) {
    const int64_t k = a.k_lo + (job >> 1);
    const int l = (int)(job & 1);
    if (k < a.k_hi) {
      if (l == 0)
        r4_row<DPLA>(a, a.lane[0], k, lane);
      else
        r4_row<DPLI>(a, a.lane[1], k, lane);
    }
  }
  if (blockIdx.x == 0) {
    __syncthreads();
    carry_frontier<4>(a);
  }
}

// Ratio 128.  Workgroup (row, slice) pools dims slice*64 .. slice*64+63 of
// row k_lo + row over all 128 tokens: 16 dim groups of 4 x 16 token groups
// of 8, merged through LDS.  It writes its 64 pooled dims to o_buf and takes
// a ticket; the last of the row's D/64 slices normalises, rotates and
// quantises the whole row.  The last slice of the first row also carries the
// frontier (all slices of that row have finished reading it by then).  With
// no row to emit, the single workgroup only carries the frontier.
template <int DPL>
__global__ void __launch_bounds__(kPoolThreads) pool_r128_kernel(PoolArgs a) {
  __shared__ float s_m[16][64], s_s[16][64], s_a[16][64];
  __shared__ int s_last;
  const LaneDev& L = a.lane[0];
  const int64_t n_rows = a.k_hi - a.k_lo;
  if (n_rows == 0) {
    carry_frontier<128>(a);
    return;
  }
  const int S = L.D / 64;
  const int64_t row = blockIdx.x / S;
  const int slice = blockIdx.x % S;
  const int64_t k = a.k_lo + row;
  const int tid = threadIdx.x;
  const int dg = tid & 15, tg = tid >> 4;
  const int c = slice * 64 + dg * 4;

  float kv[8][4], sc[8][4];
#pragma unroll
  for (int e = 0; e < 8; ++e) fetch_token<128, 4>(a, L, 128 * k + tg + 16 * e, c, kv[e], sc[e]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = sc[0][i];
#pragma unroll
    for (int e = 1; e < 8; ++e) m = fmaxf(m, sc[e][i]);
    float den = 0.f, num = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float w = expf(sc[e][i] - m);
        den += w;
        num = fmaf(w, kv[e][i], num);
      }
    }
    s_m[tg][dg * 4 + i] = m;
    s_s[tg][dg * 4 + i] = den;
    s_a[tg][dg * 4 + i] = num;
  }
  __syncthreads();
  if (tid < 64) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < 16; ++g) M = fmaxf(M, s_m[g][tid]);
    float den = 0.f, num = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const float mg = s_m[g][tid];
        if (mg != -INFINITY) {
          const float f = expf(mg - M);
          den = fmaf(s_s[g][tid], f, den);
          num = fmaf(s_a[g][tid], f, num);
        }
      }
    }
    a.o_buf[row * L.D + slice * 64 + tid] = den > 0.f ? num / den : 0.f;
    __threadfence();
    int last = 0;
    if (tid == 0) {
      const unsigned t = __hip_atomic_fetch_add(a.tickets + row, 1u, __ATOMIC_ACQ_REL,
                                                __HIP_MEMORY_SCOPE_AGENT);
      last = t == (unsigned)(S - 1);
      s_last = last;
    }
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid < 64) {
    float o[DPL];
    const float* src = a.o_buf + row * L.D + tid * DPL;
    // Acquire-ordered loads of the other slices' results.
#pragma unroll
    for (int i = 0; i < DPL; ++i)
      o[i] = __hip_atomic_load(src + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    float* pre = L.prequant ? L.prequant + row * L.D : nullptr;
    finish_row_wave<DPL>(o, L, a.n_rot, a.log2_base, a.rms_eps, k, 128, pre, L.rows + k * L.D, tid);
  }
  if (row == 0) carry_frontier<128>(a);
}

__global__ void __launch_bounds__(kPoolThreads) frontier_fill_kernel(FillArgs f) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (int l = 0; l < f.n_lanes; ++l) {
    for (int64_t i = i0; i < f.n[l]; i += stride) {
      f.kv[l][i] = 0.f;
      f.sc[l][i] = -INFINITY;
    }
  }
  if (i0 < f.n_ctrl) f.ctrl[i0] = 0u;
}

template <int A, int I>
void launch_r4(const PoolArgs& a, int64_t grid, hipStream_t s) {
  hipLaunchKernelGGL((pool_r4_kernel<A, I>), dim3((unsigned)grid), dim3(kPoolThreads), 0, s, a);
}

template <int A>
void launch_r4_a(const PoolArgs& a, int dpli, int64_t grid, hipStream_t s) {
  switch (dpli) {
    case 1: launch_r4<A, 1>(a, grid, s); break;
    case 2: launch_r4<A, 2>(a, grid, s); break;
    case 4: launch_r4<A, 4>(a, grid, s); break;
    default: launch_r4<A, 8>(a, grid, s); break;
  }
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t stream) {
  const int64_t n_rows = a.k_hi - a.k_lo;
  if (a.ratio == 4) {
    const int64_t other_jobs = (n_rows - a.n_head) * 2;
    const int64_t grid = 1 + (other_jobs + 3) / 4;
    const int dpla = a.lane[0].D / 64, dpli = a.lane[1].D / 64;
    switch (dpla) {
      case 1: launch_r4_a<1>(a, dpli, grid, stream); break;
      case 2: launch_r4_a<2>(a, dpli, grid, stream); break;
      case 4: launch_r4_a<4>(a, dpli, grid, stream); break;
      default: launch_r4_a<8>(a, dpli, grid, stream); break;
    }
  } else {
    const int S = a.lane[0].D / 64;
    const int64_t grid = n_rows == 0 ? 1 : n_rows * S;
    switch (S) {
      case 1: hipLaunchKernelGGL((pool_r128_kernel<1>), dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, a); break;
      case 2: hipLaunchKernelGGL((pool_r128_kernel<2>), dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, a); break;
      case 4: hipLaunchKernelGGL((pool_r128_kernel<4>), dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, a); break;
      default: hipLaunchKernelGGL((pool_r128_kernel<8>), dim3((unsigned)grid), dim3(kPoolThreads), 0, stream, a); break;
    }
  }
  return hipGetLastError();
}

hipError_t launch_fill(const FillArgs& f, hipStream_t stream) {
  hipLaunchKernelGGL(frontier_fill_kernel, dim3(64), dim3(kPoolThreads), 0, stream, f);
  return hipGetLastError();
}

}  // namespace ds4c
