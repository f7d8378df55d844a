// Projection GEMM: out[t, c] = sum_h x[t, h] * W[c, h] for the four weight
// blocks of a layer (wkv and wgate of each lane, Part 3 §4) written as one
// [T, N] float32 matrix.  Both operands are K-contiguous (x rows, weight rows).
//
// MFMA design for gfx950 (wave64):
//  * One 256-thread workgroup (4 waves) computes a BM x BN tile; each wave a
//    (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks with fp32 accumulators.
//    bf16 uses v_mfma_f32_32x32x16_bf16, float32 v_mfma_f32_32x32x2_f32.
//  * K advances in tiles of 128 bytes per row (64 bf16 / 32 fp32), staged
//    through LDS in 16-byte slots, double-buffered: the global loads of the
//    next K tile are in flight while the MFMAs consume the current one.
//  * Slot (row, chunk) lives at row*8 + (chunk ^ f(row)) with
//    f(row) = (row & 7) ^ ((row >> 3) & 1), so the 16-byte fragment reads of
//    8 or 16 consecutive lanes (consecutive rows, same chunk) hit distinct banks.
//  * Inside one MFMA the K order is free as long as A and B agree, so lane
//    half h reads chunk 2*kk + h of the K tile for both operands.
//  * Workgroups are dealt to the 8 XCDs round-robin; tile ids are remapped so
//    each XCD owns a contiguous range, walked in groups of GM tile-rows, which
//    keeps the x rows and weight rows an XCD reads inside its own L2.
//  * Weight rows are found per row (a tile may straddle two weight blocks).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_args.h"
#include "launch.h"

namespace ds4c {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

constexpr int kThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

template <typename Tin>
__device__ __forceinline__ void mfma_chunk(const u32x4& a, const u32x4& b, f32x16& acc);

template <>
__device__ __forceinline__ void mfma_chunk<uint16_t>(const u32x4& a, const u32x4& b, f32x16& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                acc, 0, 0, 0);
}

template <>
__device__ __forceinline__ void mfma_chunk<float>(const u32x4& a, const u32x4& b, f32x16& acc) {
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[0]), __uint_as_float(b[0]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[1]), __uint_as_float(b[1]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[2]), __uint_as_float(b[2]), acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(a[3]), __uint_as_float(b[3]), acc, 0, 0, 0);
}

// Start of weight row n of the concatenated [N, K] operand.  The blocks are
// picked with constant indices only, so the argument block stays in SGPRs.
template <typename Tin>
__device__ __forceinline__ const Tin* weight_row(const ProjArgs& a, int n) {
  const void* w = a.seg[0].w;
  int c0 = a.seg[0].col0;
  if (a.n_seg > 1 && n >= a.seg[1].col0) { w = a.seg[1].w; c0 = a.seg[1].col0; }
  if (a.n_seg > 2 && n >= a.seg[2].col0) { w = a.seg[2].w; c0 = a.seg[2].col0; }
  if (a.n_seg > 3 && n >= a.seg[3].col0) { w = a.seg[3].w; c0 = a.seg[3].col0; }
  return reinterpret_cast<const Tin*>(w) + (int64_t)(n - c0) * a.K;
}

// Global -> registers: one 16-byte chunk per staged row, K offset k0.
template <int A_PER, int B_PER, typename Tin>
__device__ __forceinline__ void gload(u32x4 (&ra)[A_PER], u32x4 (&rb)[B_PER], const Tin* const (&ap)[A_PER],
                                      const Tin* const (&bp)[B_PER], int k0) {
#pragma unroll
  for (int i = 0; i < A_PER; ++i) ra[i] = *reinterpret_cast<const u32x4*>(ap[i] + k0);
#pragma unroll
  for (int i = 0; i < B_PER; ++i) rb[i] = *reinterpret_cast<const u32x4*>(bp[i] + k0);
}

// Registers -> one LDS stage (A rows then B rows), swizzled 16-byte slots.
template <int BM, int A_PER, int B_PER>
__device__ __forceinline__ void sstore(u32x4* st, const u32x4 (&ra)[A_PER], const u32x4 (&rb)[B_PER], int t) {
  const int c = t & 7;
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    const int row = (t >> 3) + 32 * i;
    st[row * 8 + (c ^ swz(row))] = ra[i];
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    const int row = (t >> 3) + 32 * i;
    st[(BM + row) * 8 + (c ^ swz(row))] = rb[i];
  }
}

template <typename Tin, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(kThreads) proj_mfma_kernel(ProjArgs a, int tiles_m, int tiles_n, int gm) {
  constexpr int kElems = 16 / (int)sizeof(Tin);  // elements per 16-byte chunk
  constexpr int BK = 8 * kElems;                  // K elements per tile (8 chunks per row)
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int A_PER = BM * 8 / kThreads, B_PER = BN * 8 / kThreads;
  static_assert(WM * WN == 4, "four waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32x32 blocks");
  static_assert((BM * 8) % kThreads == 0 && (BN * 8) % kThreads == 0, "whole chunks per thread");
  __shared__ u32x4 smem[2][(BM + BN) * 8];

  const int t = threadIdx.x;
  if (blockIdx.x == 0)
    for (int i = t; i < a.n_zero; i += kThreads) a.zero_ptr[i] = 0u;

  // XCD-contiguous logical tile id, then grouped (GM tile-rows) order.
  const int n_tiles = tiles_m * tiles_n;
  const int b = blockIdx.x;
  const int x = b % kXcds, j = b / kXcds;
  const int q = n_tiles / kXcds, rem = n_tiles % kXcds;
  const int logical = x * q + min(x, rem) + j;
  const int group_size = gm * tiles_n;
  const int first_m = (logical / group_size) * gm;
  const int rows_in_group = min(tiles_m - first_m, gm);
  const int in_group = logical % group_size;
  const int tm = first_m + in_group % rows_in_group;
  const int tn = in_group / rows_in_group;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;

  // Global addresses of the chunks this thread stages: chunk (row, c) with
  // row = t/8 + 32*i and c = t%8.  Rows past the end are clamped (loaded,
  // never stored).
  const int c_ld = t & 7;
  const Tin* a_ptr[A_PER];
  const Tin* b_ptr[B_PER];
  const Tin* X = reinterpret_cast<const Tin*>(a.x);
#pragma unroll
  for (int i = 0; i < A_PER; ++i) {
    int64_t r = m0 + (t >> 3) + 32 * i;
    r = r < a.M ? r : a.M - 1;
    a_ptr[i] = X + r * a.K + c_ld * kElems;
  }
#pragma unroll
  for (int i = 0; i < B_PER; ++i) {
    int n = n0 + (t >> 3) + 32 * i;
    n = n < a.N ? n : a.N - 1;
    b_ptr[i] = weight_row<Tin>(a, n) + c_ld * kElems;
  }
  u32x4 ra[A_PER], rb[B_PER];

  const int wave = t >> 6, lane = t & 63;
  const int wm = wave / WN, wn = wave % WN;
  const int h = lane >> 5, r32 = lane & 31;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x16{};

  const int nk = a.K / BK;
  gload<A_PER, B_PER>(ra, rb, a_ptr, b_ptr, 0);
  sstore<BM, A_PER, B_PER>(smem[0], ra, rb, t);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int s = kt & 1;
    if (kt + 1 < nk) gload<A_PER, B_PER>(ra, rb, a_ptr, b_ptr, (kt + 1) * BK);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int c = 2 * kk + h;
      u32x4 af[FM], bfr[FN];
#pragma unroll
      for (int fm = 0; fm < FM; ++fm) {
        const int row = wm * TM + fm * 32 + r32;
        af[fm] = smem[s][row * 8 + (c ^ swz(row))];
      }
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) {
        const int row = wn * TN + fn * 32 + r32;
        bfr[fn] = smem[s][(BM + row) * 8 + (c ^ swz(row))];
      }
#pragma unroll
      for (int fm = 0; fm < FM; ++fm)
#pragma unroll
        for (int fn = 0; fn < FN; ++fn) mfma_chunk<Tin>(af[fm], bfr[fn], acc[fm][fn]);
    }
    if (kt + 1 < nk) sstore<BM, A_PER, B_PER>(smem[s ^ 1], ra, rb, t);
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column r32, rows 8*(v/4) + 4*h + v%4.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = n0 + wn * TN + fn * 32 + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * TM + fm * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < a.M && n < a.N) a.out[m * a.N + n] = acc[fm][fn][v];
      }
    }
  }
}

struct TileCfg {
  int bm, bn;
};

template <typename Tin>
void launch_cfg(const ProjArgs& a, TileCfg c, hipStream_t stream) {
  const int tiles_m = (int)((a.M + c.bm - 1) / c.bm);
  const int tiles_n = (a.N + c.bn - 1) / c.bn;
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const int gm = 4;
  if (c.bm == 256)
    hipLaunchKernelGGL((proj_mfma_kernel<Tin, 256, 160, 4, 1>), grid, dim3(kThreads), 0, stream, a, tiles_m,
                       tiles_n, gm);
  else if (c.bm == 128)
    hipLaunchKernelGGL((proj_mfma_kernel<Tin, 128, 128, 2, 2>), grid, dim3(kThreads), 0, stream, a, tiles_m,
                       tiles_n, gm);
  else
    hipLaunchKernelGGL((proj_mfma_kernel<Tin, 64, 64, 2, 2>), grid, dim3(kThreads), 0, stream, a, tiles_m,
                       tiles_n, gm);
}

}  // namespace

// Tile shape with the least work per CU: ceil(tiles / 256 CUs) rounds of
// bm*bn outputs each; ties go to the larger tile (fewer K-tile reloads).
int proj_tile_rows(int64_t M, int N) {
  const TileCfg cfgs[] = {{256, 160}, {128, 128}, {64, 64}};
  int64_t best = -1;
  int pick = 64;
  for (const TileCfg& c : cfgs) {
    const int64_t tiles = ((M + c.bm - 1) / c.bm) * ((N + c.bn - 1) / c.bn);
    const int64_t cost = ((tiles + 255) / 256) * c.bm * c.bn;
    if (best < 0 || cost < best) {
      best = cost;
      pick = c.bm;
    }
  }
  return pick;
}

hipError_t launch_proj(const ProjArgs& a, int in_dtype, hipStream_t stream) {
  const int bm = proj_tile_rows(a.M, a.N);
  const TileCfg c = bm == 256 ? TileCfg{256, 160} : bm == 128 ? TileCfg{128, 128} : TileCfg{64, 64};
  if (in_dtype == 1)
    launch_cfg<uint16_t>(a, c, stream);
  else
    launch_cfg<float>(a, c, stream);
  return hipGetLastError();
}

}  // namespace ds4c
