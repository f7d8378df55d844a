// One decode token through a compressed layer in one launch (Part 3 §4,
// compressor_decode_one; Part 3 §5, the ratio-4 frontier).
//
// Each wave computes one projected column (a dot product of a weight row
// with x) and stores it straight into the frontier row
// (coff-1)*ratio + pos%ratio, adding APE[pos%ratio] to scores.  Every
// workgroup then takes a ticket; the last one resets the ticket and, when
// (pos+1) % ratio == 0, pools the frontier into row pos/ratio of each lane
// (norm, tail RoPE, codec) and on ratio-4 layers copies rows 4..7 to 0..3.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace ds4c {

namespace {

constexpr int kDecThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// Dot product of a K-long weight row with x, one wave, 16 bytes per lane per step.
template <typename Tin>
__device__ __forceinline__ float wave_dot(const Tin* __restrict__ w, const Tin* __restrict__ x, int K, int lane);

template <>
__device__ __forceinline__ float wave_dot<uint16_t>(const uint16_t* __restrict__ w,
                                                    const uint16_t* __restrict__ x, int K, int lane) {
  float acc = 0.f;
  for (int k = lane * 8; k < K; k += kWave * 8) {
    const uint4 wv = *reinterpret_cast<const uint4*>(w + k);
    const uint4 xv = *reinterpret_cast<const uint4*>(x + k);
    acc = fmaf(bf16_lo(wv.x), bf16_lo(xv.x), acc);
    acc = fmaf(bf16_hi(wv.x), bf16_hi(xv.x), acc);
    acc = fmaf(bf16_lo(wv.y), bf16_lo(xv.y), acc);
    acc = fmaf(bf16_hi(wv.y), bf16_hi(xv.y), acc);
    acc = fmaf(bf16_lo(wv.z), bf16_lo(xv.z), acc);
    acc = fmaf(bf16_hi(wv.z), bf16_hi(xv.z), acc);
    acc = fmaf(bf16_lo(wv.w), bf16_lo(xv.w), acc);
    acc = fmaf(bf16_hi(wv.w), bf16_hi(xv.w), acc);
  }
  return wave_sum(acc);
}

template <>
__device__ __forceinline__ float wave_dot<float>(const float* __restrict__ w, const float* __restrict__ x,
                                                 int K, int lane) {
  float acc = 0.f;
  for (int k = lane * 4; k < K; k += kWave * 4) {
    const float4 wv = *reinterpret_cast<const float4*>(w + k);
    const float4 xv = *reinterpret_cast<const float4*>(x + k);
    acc = fmaf(wv.x, xv.x, acc);
    acc = fmaf(wv.y, xv.y, acc);
    acc = fmaf(wv.z, xv.z, acc);
    acc = fmaf(wv.w, xv.w, acc);
  }
  return wave_sum(acc);
}

// Running softmax-pool state of DPL dims over frontier rows [r0, r1) on
// columns c .. c+DPL-1, folded one row at a time.
template <int DPL>
__device__ __forceinline__ void pool_rows(const LaneDev& L, int r0, int r1, int c, float (&m)[DPL],
                                          float (&s)[DPL], float (&acc)[DPL]) {
  for (int r = r0; r < r1; ++r) {
    float kv[DPL], sc[DPL];
    load_vec<DPL>(kv, L.fr_kv + (int64_t)r * L.W + c);
    load_vec<DPL>(sc, L.fr_sc + (int64_t)r * L.W + c);
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      if (sc[i] == -INFINITY) continue;
      if (sc[i] > m[i]) {
        const float f = expf(m[i] - sc[i]);  // 0 when m is -inf
        s[i] = s[i] * f + 1.f;
        acc[i] = fmaf(acc[i], f, kv[i]);
        m[i] = sc[i];
      } else {
        const float w = expf(sc[i] - m[i]);
        s[i] += w;
        acc[i] = fmaf(w, kv[i], acc[i]);
      }
    }
  }
}

// Ratio-4 boundary for one lane on one wave: rows 0..3 on columns [0, D),
// rows 4..7 on columns [D, 2D).
template <int DPL>
__device__ void r4_boundary(const DecodeArgs& a, const LaneDev& L, int64_t k, int lane) {
  float m[DPL], s[DPL], acc[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) { m[i] = -INFINITY; s[i] = 0.f; acc[i] = 0.f; }
  pool_rows<DPL>(L, 0, 4, lane * DPL, m, s, acc);
  pool_rows<DPL>(L, 4, 8, L.D + lane * DPL, m, s, acc);
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) o[i] = s[i] > 0.f ? acc[i] / s[i] : 0.f;
  finish_row_wave<DPL>(o, L, a.n_rot, a.log2_base, a.rms_eps, k, 4, L.prequant, L.rows + k * L.D, lane);
}

template <typename Tin, int DPLA, int DPLI>
__global__ void __launch_bounds__(kDecThreads) decode_kernel(DecodeArgs a) {
  __shared__ float s_m[4][512], s_s[4][512], s_a[4][512];
  __shared__ int s_last;
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int r = a.ratio;
  const int coff = r == 4 ? 2 : 1;
  const int pr = (int)(a.pos % r);
  const int slot = (coff - 1) * r + pr;

  const int col = blockIdx.x * (kDecThreads / kWave) + wave;
  if (col < a.N) {
    int sg = 0;
    while (sg + 1 < a.n_seg && col >= a.seg[sg + 1].col0) ++sg;
    const int j = col - a.seg[sg].col0;
    const Tin* w = reinterpret_cast<const Tin*>(a.seg[sg].w) + (int64_t)j * a.K;
    const float v = wave_dot<Tin>(w, reinterpret_cast<const Tin*>(a.x), a.K, lane);
    if (lane == 0) {
      const LaneDev& L = a.lane[a.seg_lane[sg]];
      if (a.seg_score[sg])
        L.fr_sc[(int64_t)slot * L.W + j] = v + L.ape[(int64_t)pr * L.W + j];
      else
        L.fr_kv[(int64_t)slot * L.W + j] = v;
    }
  }
  __syncthreads();
  if (tid == 0) {
    __threadfence();
    const unsigned t = __hip_atomic_fetch_add(a.ticket, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
    s_last = t == gridDim.x - 1;
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (tid == 0) __hip_atomic_store(a.ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if ((a.pos + 1) % r != 0) return;
  const int64_t k = a.pos / r;

  if (r == 4) {
    if (wave == 0)
      r4_boundary<DPLA>(a, a.lane[0], k, lane);
    else if (wave == 1 && a.n_lanes > 1)
      r4_boundary<DPLI>(a, a.lane[1], k, lane);
    __syncthreads();
    // Half shift: rows 4..7 -> rows 0..3, full width, both tensors.
    for (int l = 0; l < a.n_lanes; ++l) {
      const LaneDev& L = a.lane[l];
      const int nv = L.W;  // floats per row
      for (int i = tid; i < 4 * nv; i += kDecThreads) {
        const int row = i / nv, c = i % nv;
        L.fr_kv[(int64_t)row * L.W + c] = L.fr_kv[(int64_t)(row + 4) * L.W + c];
        L.fr_sc[(int64_t)row * L.W + c] = L.fr_sc[(int64_t)(row + 4) * L.W + c];
      }
    }
  } else {
    // Ratio 128: four waves pool 32 rows each, merged through LDS.
    const LaneDev& L = a.lane[0];
    float m[DPLA], s[DPLA], acc[DPLA];
#pragma unroll
    for (int i = 0; i < DPLA; ++i) { m[i] = -INFINITY; s[i] = 0.f; acc[i] = 0.f; }
    pool_rows<DPLA>(L, wave * 32, wave * 32 + 32, lane * DPLA, m, s, acc);
#pragma unroll
    for (int i = 0; i < DPLA; ++i) {
      s_m[wave][lane * DPLA + i] = m[i];
      s_s[wave][lane * DPLA + i] = s[i];
      s_a[wave][lane * DPLA + i] = acc[i];
    }
    __syncthreads();
    if (wave == 0) {
      float o[DPLA];
#pragma unroll
      for (int i = 0; i < DPLA; ++i) {
        const int d = lane * DPLA + i;
        float M = -INFINITY;
        for (int g = 0; g < 4; ++g) M = fmaxf(M, s_m[g][d]);
        float den = 0.f, num = 0.f;
        if (M != -INFINITY) {
          for (int g = 0; g < 4; ++g) {
            if (s_m[g][d] == -INFINITY) continue;
            const float f = expf(s_m[g][d] - M);
            den = fmaf(s_s[g][d], f, den);
            num = fmaf(s_a[g][d], f, num);
          }
        }
        o[i] = den > 0.f ? num / den : 0.f;
      }
      finish_row_wave<DPLA>(o, L, a.n_rot, a.log2_base, a.rms_eps, k, 128, L.prequant, L.rows + k * L.D, lane);
    }
  }
}

template <typename Tin, int A>
void launch_dec_a(const DecodeArgs& a, int dpli, unsigned grid, hipStream_t s, const Timing& tm) {
  switch (dpli) {
    case 1: hipExtLaunchKernelGGL((decode_kernel<Tin, A, 1>), dim3(grid), dim3(kDecThreads), 0, s, tm.start, tm.stop, 0, a); break;
    case 2: hipExtLaunchKernelGGL((decode_kernel<Tin, A, 2>), dim3(grid), dim3(kDecThreads), 0, s, tm.start, tm.stop, 0, a); break;
    case 4: hipExtLaunchKernelGGL((decode_kernel<Tin, A, 4>), dim3(grid), dim3(kDecThreads), 0, s, tm.start, tm.stop, 0, a); break;
    default: hipExtLaunchKernelGGL((decode_kernel<Tin, A, 8>), dim3(grid), dim3(kDecThreads), 0, s, tm.start, tm.stop, 0, a); break;
  }
}

template <typename Tin>
void launch_dec(const DecodeArgs& a, unsigned grid, hipStream_t s, const Timing& tm) {
  const int dpla = a.lane[0].D / 64;
  const int dpli = a.n_lanes > 1 ? a.lane[1].D / 64 : 1;
  switch (dpla) {
    case 1: launch_dec_a<Tin, 1>(a, dpli, grid, s, tm); break;
    case 2: launch_dec_a<Tin, 2>(a, dpli, grid, s, tm); break;
    case 4: launch_dec_a<Tin, 4>(a, dpli, grid, s, tm); break;
    default: launch_dec_a<Tin, 8>(a, dpli, grid, s, tm); break;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int in_dtype, hipStream_t stream, const Timing& tm) {
  const unsigned grid = (unsigned)((a.N + 3) / 4);
  if (in_dtype == 1)
    launch_dec<uint16_t>(a, grid, stream, tm);
  else
    launch_dec<float>(a, grid, stream, tm);
  return hipGetLastError();
}

}  // namespace ds4c
