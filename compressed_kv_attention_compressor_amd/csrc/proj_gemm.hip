// Projection GEMM: out[t, c] = sum_h x[t, h] * W[c, h] for the four weight
// blocks of a layer (wkv and wgate of each lane, Part 3 §4) written as one
// [T, N] float32 matrix.  Both operands are K-contiguous (x rows, weight rows).
//
// MFMA design for gfx950 (wave64):
//  * One 256-thread workgroup (4 waves) computes a BM x BN tile; each wave a
//    (BM/WM) x (BN/WN) sub-tile of 32x32 MFMA blocks with fp32 accumulators.
//    bf16 uses v_mfma_f32_32x32x16_bf16, float32 v_mfma_f32_32x32x2_f32.
//  * K advances in tiles of 128 bytes per row (64 bf16 / 32 fp32) through a
//    3-stage LDS ring filled by direct global->LDS 16-byte loads (no VGPR
//    staging).  A K tile is issued two tiles ahead; the workgroup barrier
//    sits in the middle of a tile so the next tile's first fragments are read
//    while the current tile's last MFMAs run, and fragment registers are
//    double-buffered across the four K sub-steps of a tile.
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

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima so they do not wait).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

template <typename Tin, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(kThreads) proj_mfma_kernel(ProjArgs a, int tiles_m, int tiles_n, int gm) {
  constexpr int kElems = 16 / (int)sizeof(Tin);  // elements per 16-byte chunk
  constexpr int BK = 8 * kElems;                  // K elements per tile (8 chunks per row)
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int kWaves = kThreads / 64;
  constexpr int A_INS = BM / (8 * kWaves), B_INS = BN / (8 * kWaves);  // 8 rows per wave load
  constexpr int kStage = (BM + BN) * 8;                                  // 16-byte slots per stage
  static_assert(WM * WN == kWaves, "four waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32x32 blocks");
  static_assert(BM % (8 * kWaves) == 0 && BN % (8 * kWaves) == 0, "whole wave loads");
  __shared__ u32x4 smem[3 * kStage];

  const int t = threadIdx.x;

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

  const int wave = t >> 6, lane = t & 63;
  // Direct-to-LDS loads: a wave instruction fills 1 KiB of LDS = 8 rows x 8
  // slots, lane l landing in slot l.  Lane l of the instruction covering rows
  // r0..r0+7 therefore fetches chunk (l%8) ^ f(row) of row r0 + l/8.
  const Tin* X = reinterpret_cast<const Tin*>(a.x);
  const Tin* a_src[A_INS];
  const Tin* b_src[B_INS];
#pragma unroll
  for (int i = 0; i < A_INS; ++i) {
    const int row = (wave * A_INS + i) * 8 + (lane >> 3);
    int64_t r = m0 + row;
    r = r < a.M ? r : a.M - 1;
    a_src[i] = X + r * a.K + ((lane & 7) ^ swz(row)) * kElems;
  }
#pragma unroll
  for (int i = 0; i < B_INS; ++i) {
    const int row = (wave * B_INS + i) * 8 + (lane >> 3);
    int n = n0 + row;
    n = n < a.N ? n : a.N - 1;
    b_src[i] = weight_row<Tin>(a, n) + ((lane & 7) ^ swz(row)) * kElems;
  }
  auto issue = [&](int kt, int st) {
    const int k0 = kt * BK;
    __attribute__((address_space(3))) u32x4* base =
        (__attribute__((address_space(3))) u32x4*)(smem + st * kStage);
#pragma unroll
    for (int i = 0; i < A_INS; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(a_src[i] + k0),
                                       (__attribute__((address_space(3))) void*)(base + (wave * A_INS + i) * 64),
                                       16, 0, 0);
#pragma unroll
    for (int i = 0; i < B_INS; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(b_src[i] + k0),
                                       (__attribute__((address_space(3))) void*)(base + (BM + (wave * B_INS + i) * 8) * 8),
                                       16, 0, 0);
  };

  const int wm = wave / WN, wn = wave % WN;
  const int h = lane >> 5, r32 = lane & 31;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x16{};

  // Fragment registers, double-buffered across K sub-steps.
  u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  auto frags = [&](u32x4 (&fa)[FM], u32x4 (&fb)[FN], int st, int kk) {
    const u32x4* base = smem + st * kStage;
    const int c = 2 * kk + h;
#pragma unroll
    for (int fm = 0; fm < FM; ++fm) {
      const int row = wm * TM + fm * 32 + r32;
      fa[fm] = base[row * 8 + (c ^ swz(row))];
    }
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int row = wn * TN + fn * 32 + r32;
      fb[fn] = base[(BM + row) * 8 + (c ^ swz(row))];
    }
  };
  auto mma = [&](const u32x4 (&fa)[FM], const u32x4 (&fb)[FN]) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn) mfma_chunk<Tin>(fa[fm], fb[fn], acc[fm][fn]);
  };
  // Interleave hint: one MFMA, one LDS read, repeated, then the rest of the MFMAs.
  auto interleave = [&]() {
#pragma unroll
    for (int i = 0; i < FM + FN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FM * FN - (FM + FN) > 0 ? FM * FN - (FM + FN) : 0, 0);
  };

  const int nk = a.K / BK;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  if (nk > 1)
    wait_vm<A_INS + B_INS>();
  else
    wait_vm<0>();
  asm volatile("s_barrier" ::: "memory");
  frags(fa0, fb0, 0, 0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % 3;
    frags(fa1, fb1, st, 1);
    mma(fa0, fb0);
    interleave();
    frags(fa0, fb0, st, 2);
    mma(fa1, fb1);
    interleave();
    if (kt + 1 < nk) {
      // Tile kt+1 has landed for every wave, and every wave is done with tile
      // kt-1, whose stage the issue below refills.
      wait_vm<0>();
      asm volatile("s_barrier" ::: "memory");
      if (kt + 2 < nk) issue(kt + 2, (kt + 2) % 3);
    }
    frags(fa1, fb1, st, 3);
    mma(fa0, fb0);
    interleave();
    if (kt + 1 < nk) frags(fa0, fb0, (kt + 1) % 3, 0);
    mma(fa1, fb1);
    interleave();
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
void launch_cfg(const ProjArgs& a, TileCfg c, hipStream_t stream, const Timing& tm) {
  const int tiles_m = (int)((a.M + c.bm - 1) / c.bm);
  const int tiles_n = (a.N + c.bn - 1) / c.bn;
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const int gm = 4;
  if (c.bm == 256)
    hipExtLaunchKernelGGL((proj_mfma_kernel<Tin, 256, 160, 4, 1>), grid, dim3(kThreads), 0, stream, tm.start, tm.stop, 0, a, tiles_m,
                       tiles_n, gm);
  else if (c.bm == 128)
    hipExtLaunchKernelGGL((proj_mfma_kernel<Tin, 128, 128, 2, 2>), grid, dim3(kThreads), 0, stream, tm.start, tm.stop, 0, a, tiles_m,
                       tiles_n, gm);
  else
    hipExtLaunchKernelGGL((proj_mfma_kernel<Tin, 64, 64, 2, 2>), grid, dim3(kThreads), 0, stream, tm.start, tm.stop, 0, a, tiles_m,
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

hipError_t launch_proj(const ProjArgs& a, int in_dtype, hipStream_t stream, const Timing& tm) {
  const int bm = proj_tile_rows(a.M, a.N);
  const TileCfg c = bm == 256 ? TileCfg{256, 160} : bm == 128 ? TileCfg{128, 128} : TileCfg{64, 64};
  if (in_dtype == 1)
    launch_cfg<uint16_t>(a, c, stream, tm);
  else
    launch_cfg<float>(a, c, stream, tm);
  return hipGetLastError();
}

}  // namespace ds4c
