// One decode token through a compressed layer (Part 3 §4,
// compressor_decode_one; Part 3 §5, the ratio-4 frontier).
//
// Every token: a GEMV launch in which each wave computes two projected
// columns (dot products of weight rows with x, x staged once per workgroup in
// LDS) and stores them straight into frontier row (coff-1)*ratio + pos%ratio,
// adding APE[pos%ratio] to scores.  Only when (pos+1) % ratio == 0 a second,
// single-workgroup launch pools the frontier into row pos/ratio of each lane
// (norm, tail RoPE, codec) and on ratio-4 layers copies rows 4..7 to 0..3;
// it loads all of a lane's window entries at once, so the pool costs one
// memory round trip rather than one per row.
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

// Ratio-4 window boundary on one workgroup of SA + 1 waves: SA attention
// waves (DPLA dims per lane) and one indexer wave (DPLI per lane) load the
// window's 8 entries of their dims at once -- rows 0..3 on columns [0, D),
// rows 4..7 on columns [D, 2D) -- pool them like a prefill window, finish the
// row (the attention row's sum of squares meets in LDS), and then the whole
// workgroup copies rows 4..7 to rows 0..3.
template <int SA, int DPLA, int DPLI>
__global__ void __launch_bounds__(64 * (SA + 1)) decode_r4_finish_kernel(DecodeArgs a) {
  __shared__ float s_ss[SA];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t k = a.pos / 4;
  if (wave < SA) {
    const LaneDev& L = a.lane[0];
    const int d0 = wave * (kWave * DPLA) + lane * DPLA;
    float kv[8][DPLA], sc[8][DPLA], o[DPLA];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int c = (e < 4 ? 0 : L.D) + d0;
      load_vec<DPLA>(kv[e], L.fr_kv + e * L.W + c);
      load_vec<DPLA>(sc[e], L.fr_sc + e * L.W + c);
    }
    pool_entries<8, DPLA>(kv, sc, o);
    const float ss = wave_sum(row_sumsq<DPLA>(o));
    if (lane == 0) s_ss[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < SA; ++w) tot += s_ss[w];
    finish_row_part<DPLA>(o, L, rms_inv(tot, L.D, a.rms_eps), d0, a.n_rot, a.log2_base, k, 4, L.prequant,
                          L.rows + k * L.D, lane);
  } else {
    if (a.n_lanes > 1) {
      const LaneDev& L = a.lane[1];
      float kv[8][DPLI], sc[8][DPLI], o[DPLI];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int c = (e < 4 ? 0 : L.D) + lane * DPLI;
        load_vec<DPLI>(kv[e], L.fr_kv + e * L.W + c);
        load_vec<DPLI>(sc[e], L.fr_sc + e * L.W + c);
      }
      pool_entries<8, DPLI>(kv, sc, o);
      __syncthreads();
      finish_row_wave<DPLI>(o, L, a.n_rot, a.log2_base, a.rms_eps, k, 4, L.prequant, L.rows + k * L.D, lane);
    } else {
      __syncthreads();
    }
  }
  __syncthreads();
  // Half shift: rows 4..7 -> rows 0..3, full width, both tensors.
  for (int l = 0; l < a.n_lanes; ++l) {
    const LaneDev& L = a.lane[l];
    const int nv = L.W / 4;
    for (int i = threadIdx.x; i < 4 * nv; i += blockDim.x) {
      const int row = i / nv, c = (i % nv) * 4;
      *reinterpret_cast<float4*>(L.fr_kv + row * L.W + c) = *reinterpret_cast<const float4*>(L.fr_kv + (row + 4) * L.W + c);
      *reinterpret_cast<float4*>(L.fr_sc + row * L.W + c) = *reinterpret_cast<const float4*>(L.fr_sc + (row + 4) * L.W + c);
    }
  }
}

// Ratio-128 window boundary on one workgroup of 16 waves: wave w pools
// frontier rows 8w .. 8w+7 (two passes of four rows, each pass's loads issued
// together) into a (max, sum, weighted sum) partial per dim; the partials
// meet in LDS and wave 0 merges them and finishes the row.
template <int DPL>
__global__ void __launch_bounds__(1024) decode_r128_finish_kernel(DecodeArgs a) {
  __shared__ float s_m[16][512], s_s[16][512], s_a[16][512];
  const LaneDev& L = a.lane[0];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t k = a.pos / 128;
  const int d0 = lane * DPL;
  float m[DPL], den[DPL], num[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) { m[i] = -INFINITY; den[i] = 0.f; num[i] = 0.f; }
  // Two passes of four rows (all loads of a pass issued together), merged
  // into a running (max, sum, weighted sum).
#pragma unroll
  for (int e0 = 0; e0 < 8; e0 += 4) {
    float kv[4][DPL], sc[4][DPL];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      load_vec<DPL>(kv[e], L.fr_kv + (wave * 8 + e0 + e) * L.W + d0);
      load_vec<DPL>(sc[e], L.fr_sc + (wave * 8 + e0 + e) * L.W + d0);
    }
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      float mp = fmaxf(fmaxf(sc[0][i], sc[1][i]), fmaxf(sc[2][i], sc[3][i]));
      const float mn = fmaxf(m[i], mp);
      if (mn == -INFINITY) continue;
      const float f = expf(m[i] - mn);  // 0 when m is -inf
      den[i] *= f;
      num[i] *= f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w = expf(sc[e][i] - mn);
        den[i] += w;
        num[i] = fmaf(w, kv[e][i], num[i]);
      }
      m[i] = mn;
    }
  }
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    s_m[wave][d0 + i] = m[i];
    s_s[wave][d0 + i] = den[i];
    s_a[wave][d0 + i] = num[i];
  }
  __syncthreads();
  if (wave != 0) return;
  float o[DPL];
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const int d = d0 + i;
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < 16; ++g) M = fmaxf(M, s_m[g][d]);
    float den = 0.f, num = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int g = 0; g < 16; ++g) {
        const float mg = s_m[g][d];
        if (mg == -INFINITY) continue;
        const float f = expf(mg - M);
        den = fmaf(s_s[g][d], f, den);
        num = fmaf(s_a[g][d], f, num);
      }
    }
    o[i] = den > 0.f ? num / den : 0.f;
  }
  finish_row_wave<DPL>(o, L, a.n_rot, a.log2_base, a.rms_eps, k, 128, L.prequant, L.rows + k * L.D, lane);
}

template <int SA, int DPLA>
void launch_r4_fin(const DecodeArgs& a, int dpli, hipStream_t s, const Timing& tm) {
  const dim3 g(1), b(64 * (SA + 1));
  switch (dpli) {
    case 1: hipExtLaunchKernelGGL((decode_r4_finish_kernel<SA, DPLA, 1>), g, b, 0, s, nullptr, tm.stop, 0, a); break;
    case 2: hipExtLaunchKernelGGL((decode_r4_finish_kernel<SA, DPLA, 2>), g, b, 0, s, nullptr, tm.stop, 0, a); break;
    case 4: hipExtLaunchKernelGGL((decode_r4_finish_kernel<SA, DPLA, 4>), g, b, 0, s, nullptr, tm.stop, 0, a); break;
    default: hipExtLaunchKernelGGL((decode_r4_finish_kernel<SA, DPLA, 8>), g, b, 0, s, nullptr, tm.stop, 0, a); break;
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
    if (a.ratio == 4) {
      // Attention rows split over waves of 128 dims (64 below 128), as in prefill.
      const int dpli = a.n_lanes > 1 ? a.lane[1].D / 64 : 1;
      switch (a.lane[0].D) {
        case 64: launch_r4_fin<1, 1>(a, dpli, stream, tm); break;
        case 128: launch_r4_fin<1, 2>(a, dpli, stream, tm); break;
        case 256: launch_r4_fin<2, 2>(a, dpli, stream, tm); break;
        default: launch_r4_fin<4, 2>(a, dpli, stream, tm); break;
      }
    } else {
      const dim3 g(1), b(1024);
      switch (a.lane[0].D / 64) {
        case 1: hipExtLaunchKernelGGL((decode_r128_finish_kernel<1>), g, b, 0, stream, nullptr, tm.stop, 0, a); break;
        case 2: hipExtLaunchKernelGGL((decode_r128_finish_kernel<2>), g, b, 0, stream, nullptr, tm.stop, 0, a); break;
        case 4: hipExtLaunchKernelGGL((decode_r128_finish_kernel<4>), g, b, 0, stream, nullptr, tm.stop, 0, a); break;
        default: hipExtLaunchKernelGGL((decode_r128_finish_kernel<8>), g, b, 0, stream, nullptr, tm.stop, 0, a); break;
      }
    }
  }
  return hipGetLastError();
}

}  // namespace ds4c
