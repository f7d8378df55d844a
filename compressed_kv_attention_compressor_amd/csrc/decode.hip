// One decode token through a compressed layer (Part 3 §4,
// compressor_decode_one; Part 3 §5, the ratio-4 frontier).
//
// Every token: a GEMV launch in which each wave computes two projected
// columns (dot products of weight rows with x, x staged once per workgroup in
// LDS) and stores them straight into frontier row (coff-1)*ratio + pos%ratio,
// adding APE[pos%ratio] to scores.  Only when (pos+1) % ratio == 0 a second,
// single-workgroup launch pools the frontier into row pos/ratio of each lane
// (norm, tail RoPE, codec) and on ratio-4 layers copies rows 4..7 to 0..3.
// The launch boundary orders the pool after every column store.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace ds4c {

namespace {

constexpr int kDecThreads = 256;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

constexpr int kColsPerWave = 2;

// Two dot products of K-long weight rows with x (in LDS), one wave, 16 bytes
// per lane per step of each row.
template <typename Tin>
__device__ __forceinline__ void wave_dot2(const Tin* __restrict__ w0, const Tin* __restrict__ w1,
                                          const Tin* __restrict__ xs, int K, int lane, float* d0, float* d1);

template <>
__device__ __forceinline__ void wave_dot2<uint16_t>(const uint16_t* __restrict__ w0, const uint16_t* __restrict__ w1,
                                                    const uint16_t* __restrict__ xs, int K, int lane, float* d0,
                                                    float* d1) {
  float a0 = 0.f, a1 = 0.f;
  for (int k = lane * 8; k < K; k += kWave * 8) {
    const uint4 xv = *reinterpret_cast<const uint4*>(xs + k);
    const uint4 u = *reinterpret_cast<const uint4*>(w0 + k);
    const uint4 v = *reinterpret_cast<const uint4*>(w1 + k);
    const float x0 = bf16_lo(xv.x), x1 = bf16_hi(xv.x), x2 = bf16_lo(xv.y), x3 = bf16_hi(xv.y);
    const float x4 = bf16_lo(xv.z), x5 = bf16_hi(xv.z), x6 = bf16_lo(xv.w), x7 = bf16_hi(xv.w);
    a0 = fmaf(bf16_lo(u.x), x0, a0); a0 = fmaf(bf16_hi(u.x), x1, a0);
    a0 = fmaf(bf16_lo(u.y), x2, a0); a0 = fmaf(bf16_hi(u.y), x3, a0);
    a0 = fmaf(bf16_lo(u.z), x4, a0); a0 = fmaf(bf16_hi(u.z), x5, a0);
    a0 = fmaf(bf16_lo(u.w), x6, a0); a0 = fmaf(bf16_hi(u.w), x7, a0);
    a1 = fmaf(bf16_lo(v.x), x0, a1); a1 = fmaf(bf16_hi(v.x), x1, a1);
    a1 = fmaf(bf16_lo(v.y), x2, a1); a1 = fmaf(bf16_hi(v.y), x3, a1);
    a1 = fmaf(bf16_lo(v.z), x4, a1); a1 = fmaf(bf16_hi(v.z), x5, a1);
    a1 = fmaf(bf16_lo(v.w), x6, a1); a1 = fmaf(bf16_hi(v.w), x7, a1);
  }
  *d0 = wave_sum(a0);
  *d1 = wave_sum(a1);
}

template <>
__device__ __forceinline__ void wave_dot2<float>(const float* __restrict__ w0, const float* __restrict__ w1,
                                                 const float* __restrict__ xs, int K, int lane, float* d0, float* d1) {
  float a0 = 0.f, a1 = 0.f;
  for (int k = lane * 4; k < K; k += kWave * 4) {
    const float4 xv = *reinterpret_cast<const float4*>(xs + k);
    const float4 u = *reinterpret_cast<const float4*>(w0 + k);
    const float4 v = *reinterpret_cast<const float4*>(w1 + k);
    a0 = fmaf(u.x, xv.x, a0); a0 = fmaf(u.y, xv.y, a0); a0 = fmaf(u.z, xv.z, a0); a0 = fmaf(u.w, xv.w, a0);
    a1 = fmaf(v.x, xv.x, a1); a1 = fmaf(v.y, xv.y, a1); a1 = fmaf(v.z, xv.z, a1); a1 = fmaf(v.w, xv.w, a1);
  }
  *d0 = wave_sum(a0);
  *d1 = wave_sum(a1);
}

// Weight row of projected column col, and where its value goes.
template <typename Tin>
__device__ __forceinline__ void column_target(const DecodeArgs& a, int col, int slot, int pr, const Tin** w,
                                              float** dst, const float** ape_row) {
  int sg = 0;
  if (a.n_seg > 1 && col >= a.seg[1].col0) sg = 1;
  if (a.n_seg > 2 && col >= a.seg[2].col0) sg = 2;
  if (a.n_seg > 3 && col >= a.seg[3].col0) sg = 3;
  const ProjSeg& S = a.seg[sg];
  const int j = col - S.col0;
  const LaneDev& L = a.lane[sg >> 1];
  *w = reinterpret_cast<const Tin*>(S.w) + (int64_t)j * a.K;
  if (sg & 1) {
    *dst = L.fr_sc + (int64_t)slot * L.W + j;
    *ape_row = L.ape + (int64_t)pr * L.W + j;
  } else {
    *dst = L.fr_kv + (int64_t)slot * L.W + j;
    *ape_row = nullptr;
  }
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

// Projection of one token into its frontier row.  Workgroup b covers
// columns [8b, 8b+8), two per wave.
template <typename Tin>
__global__ void __launch_bounds__(kDecThreads) decode_gemv_kernel(DecodeArgs a) {
  extern __shared__ __align__(16) unsigned char s_x_raw[];
  Tin* s_x = reinterpret_cast<Tin*>(s_x_raw);
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const Tin* x = reinterpret_cast<const Tin*>(a.x);
  constexpr int kVec = 16 / (int)sizeof(Tin);
  for (int k = tid * kVec; k < a.K; k += kDecThreads * kVec)
    *reinterpret_cast<uint4*>(s_x + k) = *reinterpret_cast<const uint4*>(x + k);
  __syncthreads();
  const int r = a.ratio;
  const int pr = (int)(a.pos % r);
  const int slot = (r == 4 ? r : 0) + pr;
  const int c0 = (blockIdx.x * (kDecThreads / kWave) + wave) * kColsPerWave;
  if (c0 >= a.N) return;  // N is a multiple of 64: both columns exist
  const Tin *w0, *w1;
  float *d0, *d1;
  const float *ape0, *ape1;
  column_target<Tin>(a, c0, slot, pr, &w0, &d0, &ape0);
  column_target<Tin>(a, c0 + 1, slot, pr, &w1, &d1, &ape1);
  float v0, v1;
  wave_dot2<Tin>(w0, w1, s_x, a.K, lane, &v0, &v1);
  if (lane == 0) {
    *d0 = ape0 ? v0 + *ape0 : v0;
    *d1 = ape1 ? v1 + *ape1 : v1;
  }
}

// Pool at a window boundary, on one workgroup: ratio 4 pools each lane on a
// wave and then shifts; ratio 128 pools 32 rows per wave, merged in LDS.
template <int DPLA, int DPLI>
__global__ void __launch_bounds__(kDecThreads) decode_finish_kernel(DecodeArgs a) {
  __shared__ float s_m[4][512], s_s[4][512], s_a[4][512];
  const int tid = threadIdx.x;
  const int wave = tid / kWave, lane = tid % kWave;
  const int r = a.ratio;
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
      const int nv = L.W / 4;
      for (int i = tid; i < 4 * nv; i += kDecThreads) {
        const int row = i / nv, c = (i % nv) * 4;
        *reinterpret_cast<float4*>(L.fr_kv + row * L.W + c) =
            *reinterpret_cast<const float4*>(L.fr_kv + (row + 4) * L.W + c);
        *reinterpret_cast<float4*>(L.fr_sc + row * L.W + c) =
            *reinterpret_cast<const float4*>(L.fr_sc + (row + 4) * L.W + c);
      }
    }
  } else {
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

template <int A>
void launch_fin_a(const DecodeArgs& a, int dpli, hipStream_t s, const Timing& tm) {
  const dim3 g(1), b(kDecThreads);
  switch (dpli) {
    case 1: hipExtLaunchKernelGGL((decode_finish_kernel<A, 1>), g, b, 0, s, nullptr, tm.stop, 0, a); break;
    case 2: hipExtLaunchKernelGGL((decode_finish_kernel<A, 2>), g, b, 0, s, nullptr, tm.stop, 0, a); break;
    case 4: hipExtLaunchKernelGGL((decode_finish_kernel<A, 4>), g, b, 0, s, nullptr, tm.stop, 0, a); break;
    default: hipExtLaunchKernelGGL((decode_finish_kernel<A, 8>), g, b, 0, s, nullptr, tm.stop, 0, a); break;
  }
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int in_dtype, hipStream_t stream, const Timing& tm) {
  const bool boundary = (a.pos + 1) % a.ratio == 0;
  const unsigned grid = (unsigned)((a.N + kColsPerWave * 4 - 1) / (kColsPerWave * 4));
  const size_t lds = (size_t)a.K * (in_dtype == 1 ? 2 : 4);
  hipEvent_t stop = boundary ? nullptr : tm.stop;
  if (in_dtype == 1)
    hipExtLaunchKernelGGL(decode_gemv_kernel<uint16_t>, dim3(grid), dim3(kDecThreads), (uint32_t)lds, stream, tm.start,
                          stop, 0, a);
  else
    hipExtLaunchKernelGGL(decode_gemv_kernel<float>, dim3(grid), dim3(kDecThreads), (uint32_t)lds, stream, tm.start,
                          stop, 0, a);
  if (boundary) {
    const int dpla = a.lane[0].D / 64;
    const int dpli = a.n_lanes > 1 ? a.lane[1].D / 64 : 1;
    switch (dpla) {
      case 1: launch_fin_a<1>(a, dpli, stream, tm); break;
      case 2: launch_fin_a<2>(a, dpli, stream, tm); break;
      case 4: launch_fin_a<4>(a, dpli, stream, tm); break;
      default: launch_fin_a<8>(a, dpli, stream, tm); break;
    }
  }
  return hipGetLastError();
}

}  // namespace ds4c
