// Projection GEMM: out[t, c] = sum_h x[t, h] * W[c, h] for the four weight
// blocks of a layer (wkv and wgate of each lane, Part 3 §4) written as one
// [T, N] float32 matrix.  Both operands are K-contiguous (x rows, weight rows).
//
// MFMA design for gfx950 (wave64), three kernels sharing these rules:
//  * 32x32 output blocks with fp32 accumulators: bf16 inputs use
//    v_mfma_f32_32x32x16_bf16, float32 inputs v_mfma_f32_32x32x2_f32.
//  * Operand rows reach LDS through buffer loads that write LDS directly
//    (16 bytes per lane, no VGPR staging).  The buffer form matters: the
//    flat/global form counts as an LDS access too, and while one is in
//    flight every wait for LDS fragment data degenerates to a full drain.
//  * The loop bodies have no branches (loads past the last K tile re-read
//    the last tile into a buffer nothing reads again), so the compiler's
//    wait counts stay exact; issue order inside a K sub-step is pinned:
//    MFMA, fragment read for a later sub-step, and loads spread between.
//  * Inside one MFMA the K order is free as long as both operands agree, so
//    lane half h reads chunk 2*kk + h of a row's K tile for x and weights.
//  * Workgroups are dealt to the 8 XCDs round-robin; tile ids are remapped so
//    each XCD owns a contiguous range, walked in groups of GM tile-rows, which
//    keeps the x rows and weight rows an XCD reads inside its own L2.
//  * A weight tile may straddle two weight blocks; blocks start at multiples
//    of 16 columns, so each load instruction stays inside one block.
//
// proj_splitk_kernel (256 x 160 tiles, one per CU at 4096 x 2560): eight
// waves, two per SIMD, split the four K sub-steps of each 64-column K tile
// (128-byte rows, 3-stage ring); the partial sums are combined through LDS.
// With a fused epilogue it pools ratio-4 windows.
// proj_r128_splitk4_kernel (128 x 128 tiles, a call on ratio-128 window
// boundaries): eight waves, a four-way split of K over 128 x 64 wave blocks
// (128-byte rows, 4-stage ring); one tile is one window, pooled in the
// epilogue.
// proj_mfma_kernel (128 x 128 and 64 x 64 tiles, plain output): four waves,
// 32-column K stages (64-byte rows) in a 6-stage ring, loads issued five
// stages ahead.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "kernel_args.h"
#include "launch.h"

namespace ds4c {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk
typedef float f32x4 __attribute__((ext_vector_type(4)));     // four fp32 partial sums

constexpr int kThreads = 256;
constexpr int kXcds = 8;

__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }
// 64-byte rows (4 chunks): (row % 4, slot) is distinct over any 16 consecutive
// rows and (row % 2, slot) over any 8, so fragment reads are conflict free.
__device__ __forceinline__ int swz4(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

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

// Wait until at most N vector-memory operations of this wave are in flight
// (gfx9 s_waitcnt encoding: vmcnt in bits 3:0 and 15:14, expcnt and lgkmcnt
// left at their maxima so they do not wait).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// The same, and until every LDS access of this wave has completed.
template <int N>
__device__ __forceinline__ void wait_vm_lds() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}

// One 16-byte-per-lane load into LDS through a buffer descriptor over
// [base, base + bytes); lane l's data lands at lds + 16*l.
__device__ __forceinline__ void load_lds16(const void* base, int bytes, __attribute__((address_space(3))) void* lds,
                                           uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(__builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000),
                                           lds, 16, voff, soff, 0, 0);
}



// LDS index of element (row, col) of a 128 x 128 fp32 tile, column-major:
// a column's 128 rows are 32 groups of 4 consecutive rows (16 bytes), group
// G at slot (G & 16) | ((G ^ 2 col ^ col / 8 ^ G / 16) mod 16).  Both the
// accumulator stores (one group of 16 consecutive columns) and the pool's
// reads (8 groups of 2 adjacent columns) then touch 16 different bank groups
// per 16 lanes.
__device__ __forceinline__ int tile128_ix(int row, int col) {
  const int g = row >> 2;
  return col * 128 + (((g ^ (col << 1) ^ (col >> 3) ^ (g >> 4)) & 15) | (g & 16)) * 4 + (row & 3);
}

template <typename Tin, int BM, int BN, int WM, int WN>
__global__ void __launch_bounds__(kThreads) proj_mfma_kernel(ProjArgs a, int tiles_m, int tiles_n, int gm) {
  constexpr int kElems = 16 / (int)sizeof(Tin);  // elements per 16-byte chunk
  constexpr int kElemBytes = (int)sizeof(Tin);
  constexpr int BK = 4 * kElems;                  // K elements per stage (4 chunks = 64 bytes per row)
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int kWaves = kThreads / 64;
  constexpr int kRows = BM + BN;
  constexpr int kInsA = BM / 16, kInsB = BN / 16;  // 16 rows x 64 bytes per load instruction
  constexpr int kDmaA = (kInsA + kWaves - 1) / kWaves, kDmaB = (kInsB + kWaves - 1) / kWaves;
  constexpr int kDma = kDmaA + kDmaB;             // load instructions per wave per stage
  constexpr int kNst = 6;                         // LDS stages
  constexpr int kLead = kNst - 1;                 // stages issued ahead
  constexpr int kStage = kRows * 4;               // 16-byte slots per stage
  static_assert(WM * WN == kWaves, "four waves");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "32x32 blocks");
  static_assert(BM % 16 == 0 && BN % 16 == 0, "whole 16-row loads");
  __shared__ u32x4 smem[kNst * kStage];

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

  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;

  // Loads: instruction `ins` fills stage rows 16*ins .. 16*ins+15 (rows < BM
  // are x rows m0 + r, the rest weight rows n0 + r - BM); lane l lands in
  // slot l of the instruction's 1 KiB, i.e. row 16*ins + l/4, slot l%4, and
  // so fetches logical chunk (l%4) ^ f(row).  A wave's first kDmaA
  // instructions cover x rows, the rest weight rows; a wave without a k-th
  // instruction of a kind repeats the last one (same bytes, same slots).
  const int64_t rows_left = a.M - m0;  // >= 1
  const char* x_base = reinterpret_cast<const char*>(a.x) + m0 * a.K * kElemBytes;
  const int x_bytes = (int)((rows_left < BM ? rows_left : BM) * a.K * kElemBytes);
  const void* l_base[kDma];
  int l_bytes[kDma];
  uint32_t l_off[kDma];
  int l_slot[kDma];
#pragma unroll
  for (int i = 0; i < kDmaA; ++i) {
    const int ins = min(wave + kWaves * i, kInsA - 1);
    l_slot[i] = ins * 64;
    const int row = ins * 16 + (lane >> 2);
    const int r = row < rows_left ? row : (int)rows_left - 1;
    l_base[i] = x_base;
    l_bytes[i] = x_bytes;
    l_off[i] = (uint32_t)((r * a.K + ((lane & 3) ^ swz4(row)) * kElems) * kElemBytes);
  }
#pragma unroll
  for (int i = 0; i < kDmaB; ++i) {
    const int ins = min(wave + kWaves * i, kInsB - 1);
    l_slot[kDmaA + i] = (kInsA + ins) * 64;
    const int row = BM + ins * 16 + (lane >> 2);
    // Weight blocks start at multiples of 16 columns, so the 16 rows of an
    // instruction share a block; rows past N repeat row N-1.
    int n_first = n0 + ins * 16;
    n_first = n_first < a.N ? n_first : a.N - 1;
    int n = n0 + row - BM;
    n = n < a.N ? n : a.N - 1;
    const void* w = a.seg[0].w;
    int c0 = a.seg[0].col0, cn = a.seg[0].n;
    if (a.n_seg > 1 && n_first >= a.seg[1].col0) { w = a.seg[1].w; c0 = a.seg[1].col0; cn = a.seg[1].n; }
    if (a.n_seg > 2 && n_first >= a.seg[2].col0) { w = a.seg[2].w; c0 = a.seg[2].col0; cn = a.seg[2].n; }
    if (a.n_seg > 3 && n_first >= a.seg[3].col0) { w = a.seg[3].w; c0 = a.seg[3].col0; cn = a.seg[3].n; }
    l_base[kDmaA + i] = w;
    l_bytes[kDmaA + i] = cn * a.K * kElemBytes;
    l_off[kDmaA + i] = (uint32_t)(((n - c0) * a.K + ((lane & 3) ^ swz4(row)) * kElems) * kElemBytes);
  }
  // K range of this workgroup: split blockIdx.y of a.k_split covers columns
  // k0 .. k0 + a.k_len - 1 and writes its own output plane.
  const int k0 = (int)blockIdx.y * a.k_len;
  const int nh = a.k_len / BK;  // stages along K (even)
  // Load instructions i0 .. i0+cnt-1 of stage `hs` (clamped to the last one).
  auto issue = [&](int hs, int i0, int cnt) {
    const int hc = min(hs, nh - 1);
    const uint32_t soff = (uint32_t)((k0 + hc * BK) * kElemBytes);
    __attribute__((address_space(3))) u32x4* base =
        (__attribute__((address_space(3))) u32x4*)(smem + (hs % kNst) * kStage);
#pragma unroll
    for (int i = 0; i < kDma; ++i)
      if (i >= i0 && i < i0 + cnt)
        load_lds16(l_base[i], l_bytes[i], (__attribute__((address_space(3))) void*)(base + l_slot[i]), l_off[i], soff);
  };

  const int wm = wave / WN, wn = wave % WN;
  const int h = lane >> 5, r32 = lane & 31;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x16{};

  // Fragment registers: one set per K sub-step of two consecutive stages,
  // read one stage (two sub-steps) ahead.
  u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN], fa2[FM], fb2[FN], fa3[FM], fb3[FN];
  // Fragment f (0..FM+FN-1: x blocks, then weight blocks) of sub-step kk of stage hs.
  auto frag = [&](u32x4 (&fa)[FM], u32x4 (&fb)[FN], int f, int hs, int kk) {
    const u32x4* base = smem + (hs % kNst) * kStage;
    const int c = 2 * kk + h;
    if (f < FM) {
      const int row = wm * TM + f * 32 + r32;
      fa[f] = base[row * 4 + (c ^ swz4(row))];
    } else {
      const int row = BM + wn * TN + (f - FM) * 32 + r32;
      fb[f - FM] = base[row * 4 + (c ^ swz4(row))];
    }
  };
  auto frags = [&](u32x4 (&fa)[FM], u32x4 (&fb)[FN], int hs, int kk) {
#pragma unroll
    for (int f = 0; f < FM + FN; ++f) frag(fa, fb, f, hs, kk);
  };
  // One K sub-step in a fixed issue order: MFMA i, then (for the first FM+FN)
  // fragment i of the sub-step two ahead, then (spread evenly) one of the nd
  // loads i0.. of stage hs+kLead.
  auto sub_step = [&](const u32x4 (&ca)[FM], const u32x4 (&cb)[FN], u32x4 (&na)[FM], u32x4 (&nb)[FN], int hs_next,
                      int kk_next, int hs_load, int i0, int nd) {
    constexpr int kM = FM * FN, kR = FM + FN;
    int d = 0;
#pragma unroll
    for (int i = 0; i < kM; ++i) {
      mfma_chunk<Tin>(ca[i / FN], cb[i % FN], acc[i / FN][i % FN]);
      if (i < kR) frag(na, nb, i, hs_next, kk_next);
      if (nd > 0 && (i * nd) / kM != ((i + 1) * nd) / kM) {
        issue(hs_load, i0 + d, 1);
        ++d;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Fewer MFMAs than fragments or loads (small tiles): issue the rest.
#pragma unroll
    for (int f = kM; f < kR; ++f) frag(na, nb, f, hs_next, kk_next);
    for (; d < nd; ++d) issue(hs_load, i0 + d, 1);
  };
  constexpr int kD0 = kDma / 2, kD1 = kDma - kDma / 2;  // loads per sub-step
  // Stage hs: barrier, then its two sub-steps with the next stage's fragment
  // reads and stage hs+kLead's loads interleaved.  At the barrier the loads
  // of stage hs+1 have landed for every wave (the kDma*(kLead-2) issued
  // after them may be in flight), and every wave has finished reading stage
  // hs-1, which this stage's loads refill.
  auto stage = [&](int hs, const u32x4 (&ca)[FM], const u32x4 (&cb)[FN], const u32x4 (&da)[FM], const u32x4 (&db)[FN],
                   u32x4 (&na)[FM], u32x4 (&nb)[FN], u32x4 (&ma)[FM], u32x4 (&mb)[FN]) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm<kDma * (kLead - 2)>();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    sub_step(ca, cb, na, nb, hs + 1, 0, hs + kLead, 0, kD0);
    sub_step(da, db, ma, mb, hs + 1, 1, hs + kLead, kD0, kD1);
  };

#pragma unroll
  for (int hs = 0; hs < kLead; ++hs) issue(hs, 0, kDma);
  wait_vm<kDma * (kLead - 1)>();
  asm volatile("s_barrier" ::: "memory");
  frags(fa0, fb0, 0, 0);
  frags(fa1, fb1, 0, 1);
  for (int hs = 0; hs < nh; hs += 2) {
    stage(hs, fa0, fb0, fa1, fb1, fa2, fb2, fa3, fb3);
    stage(hs + 1, fa2, fb2, fa3, fb3, fa0, fb0, fa1, fb1);
  }
  wait_vm<0>();  // no LDS-bound load may outlive the loop

  // 32x32 accumulator layout: lane holds column r32, rows 8*(v/4) + 4*h + v%4.
  float* out = a.out + (int64_t)blockIdx.y * a.split_stride;
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) {
      const int n = n0 + wn * TN + fn * 32 + r32;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t m = m0 + wm * TM + fm * 32 + 8 * (v >> 2) + 4 * h + (v & 3);
        if (m < a.M && n < a.N) out[m * a.N + n] = acc[fm][fn][v];
      }
    }
  }
}


// ---------------------------------------------------------------------------
// Fused ratio-4 epilogue (Part 3 §4-§5) of a 256-token x 40-dim tile (see
// FuseArgs for the column runs).  The two wave groups' partial sums meet in
// an LDS copy of the tile (column-major, below); then each (window, dim) of
// the tile is pooled:
// window g >= 1 of the tile from its own rows as one 8-entry softmax, window
// 0's current half and the next tile's window 0 previous half as (max, sum,
// weighted sum) partials.  The tokens the frontier keeps are staged in the
// plain column layout with APE added to their scores.
// ---------------------------------------------------------------------------
// LDS index of tile element (row, col), column-major: a column's 256 rows
// are 64 groups of 4 consecutive rows (16 bytes each); group G sits at slot
// G with its low four bits XORed with col % 16.  An accumulator store (one
// 4-row group of 16 consecutive columns per 16 lanes) then touches 16
// different bank groups, and the pool's reads (one group of each of its
// dims' columns) at most two lanes per bank group; both move 16 bytes per
// lane per instruction.
__device__ __forceinline__ int tile_ix(int row, int col) {
  return col * 256 + ((((row >> 2) ^ col) & 15) | ((row >> 2) & ~15)) * 4 + (row & 3);
}

// e^(s - m) as 2^(s*log2(e) - m*log2(e)) with ml = m*log2(e): one FMA and
// the hardware base-2 exponential per weight (the epilogue's pool is bound
// by VALU issue, so the subtraction is folded into the scaling).
constexpr float kLog2e = 1.44269504088896341f;
__device__ __forceinline__ float exp_shifted(float s, float ml) {
  return __builtin_amdgcn_exp2f(fmaf(s, kLog2e, -ml));
}

// (max, sum, weighted sum) of four entries of one dim, without branches: an
// all-empty half (every score -inf) gives (-inf, 0, 0).
struct Part3 {
  float m, s, w;
};
__device__ __forceinline__ Part3 half_pool(const float (&kv)[4], const float (&sc)[4]) {
  Part3 p;
  p.m = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
  const float ml = (p.m == -INFINITY ? 0.f : p.m) * kLog2e;
  p.s = 0.f;
  p.w = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = exp_shifted(sc[e], ml);
    p.s += x;
    p.w = fmaf(x, kv[e], p.w);
  }
  return p;
}

// Softmax pool of one dim over a whole window: previous half (kp, sp) and
// current half (kc, sc).  An all-empty window gives 0.  The quotient uses
// the hardware reciprocal (about 1 ulp), well inside the pooled values'
// tolerance and below the FP8 grid the row is rounded to afterwards.
__device__ __forceinline__ float window_pool(const float (&kp)[4], const float (&sp)[4], const float (&kc)[4],
                                             const float (&sc)[4]) {
  const float m =
      fmaxf(fmaxf(fmaxf(sp[0], sp[1]), fmaxf(sp[2], sp[3])), fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
  const float ml = (m == -INFINITY ? 0.f : m) * kLog2e;
  float den = 0.f, num = 0.f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = exp_shifted(sp[e], ml);
    den += x;
    num = fmaf(x, kp[e], num);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float x = exp_shifted(sc[e], ml);
    den += x;
    num = fmaf(x, kc[e], num);
  }
  return den > 0.f ? num * __builtin_amdgcn_rcpf(den) : 0.f;
}

template <int WM, int FN>
__device__ __forceinline__ void fused_r4_epilogue(const ProjArgs& a, f32x16 (&acc)[2][FN], float* tile, int tm, int tn,
                                                  int wq, int grp, int lane) {
  const FuseArgs& f = a.fuse;
  const int h = lane >> 5, r32 = lane & 31;
  // Thread t < 480 pools dim 40*tn + t % 40 below; its APE values are read
  // first so that their latency hides behind the combine.
  const int dd = threadIdx.x % 40, rg = threadIdx.x / 40;
  const int dim = tn * 40 + dd;
  const bool pools = threadIdx.x < 480 && dim < f.d_tot;
  const int l = dim < f.d_attn ? 0 : 1;
  const int ld = dim - (l ? f.d_attn : 0), dl = l ? f.d_idx : f.d_attn, W = f.W[l];
  const int ldc = pools ? ld : 0;  // in-bounds address for every thread
  float ape_p[4], ape_c[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    ape_p[e] = f.ape[l][e * W + ldc];
    ape_c[e] = f.ape[l][e * W + dl + ldc];
  }

  // The two groups' partial sums meet: group g parks its partial of block
  // fm = 1 - g lane-major (conflict free) in LDS half g, adds the other
  // group's partial of block fm = g from half 1 - g, and stores the finished
  // block into the tile.  Each element takes exactly one addition, so the
  // result does not depend on which group owns it.
  // 32x32 accumulator layout: lane holds column r32, rows 8*(v/4) + 4*h + v%4.
  // Parked in 16-byte chunks (four consecutive v), lane-major.
  f32x4* tile4 = reinterpret_cast<f32x4*>(tile);
  constexpr int kPark4 = 4 * FN * 4 * 64;  // chunks parked per group
  asm volatile("s_barrier" ::: "memory");  // every wave is done with the ring the tile overlaps
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    if (fm == grp) continue;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        tile4[grp * kPark4 + ((wq * FN + fn) * 4 + j) * 64 + lane] =
            f32x4{acc[fm][fn][4 * j], acc[fm][fn][4 * j + 1], acc[fm][fn][4 * j + 2], acc[fm][fn][4 * j + 3]};
  }
  __syncthreads();
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    if (fm != grp) continue;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 p = tile4[(1 - grp) * kPark4 + ((wq * FN + fn) * 4 + j) * 64 + lane];
        acc[fm][fn][4 * j] += p.x;
        acc[fm][fn][4 * j + 1] += p.y;
        acc[fm][fn][4 * j + 2] += p.z;
        acc[fm][fn][4 * j + 3] += p.w;
      }
  }
  __syncthreads();
  // Rows 8j + 4h .. 8j + 4h + 3 of a 32-row block are one 4-row group.
#pragma unroll
  for (int fm = 0; fm < 2; ++fm) {
    if (fm != grp) continue;
#pragma unroll
    for (int fn = 0; fn < FN; ++fn)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        tile4[tile_ix(wq * 64 + fm * 32 + 8 * j + 4 * h, fn * 32 + r32) >> 2] =
            f32x4{acc[fm][fn][4 * j], acc[fm][fn][4 * j + 1], acc[fm][fn][4 * j + 2], acc[fm][fn][4 * j + 3]};
  }
  __syncthreads();

  const int64_t t0 = (int64_t)tm * 256;  // call-relative token of tile row 0
  const int64_t j0 = (int64_t)tm * 64;   // window of tile group 0
  // Thread t < 480 owns dim 40*tn + t % 40 and the 4-row groups [g_lo, g_hi)
  // of range t / 40 (twelve ranges of five or six groups).  Group g holds
  // the current half of window g and the previous half of window g + 1, so
  // each group is read once: window g pools the previous half kept from
  // group g - 1 with group g's current half.
  if (pools) {
    const int g_lo = rg * 64 / 12, g_hi = (rg + 1) * 64 / 12;
    float kp[4], sp[4];  // previous half of the next window
    if (g_lo > 0) {
      const f32x4 k4 = tile4[tile_ix(4 * (g_lo - 1), dd) >> 2];
      const f32x4 s4 = tile4[tile_ix(4 * (g_lo - 1), 80 + dd) >> 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kp[e] = k4[e];
        sp[e] = s4[e] + ape_p[e];
      }
    } else {
      // Window j0: its previous half lies in the previous tile (or, for
      // tile 0, in rows 0..3 of the incoming frontier, whose scores already
      // hold their APE), so both halves are written as partials.
      float kc[4], sc[4];
      const f32x4 kc4 = tile4[tile_ix(0, 40 + dd) >> 2], sc4 = tile4[tile_ix(0, 120 + dd) >> 2];
      const f32x4 kp4 = tile4[tile_ix(0, dd) >> 2], sp4 = tile4[tile_ix(0, 80 + dd) >> 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kc[e] = kc4[e];
        sc[e] = sc4[e] + ape_c[e];
        kp[e] = kp4[e];
        sp[e] = sp4[e] + ape_p[e];
      }
      if (j0 < f.n_emit) {
        const Part3 pc = half_pool(kc, sc);
        float* q = f.part + ((int64_t)tm * 2 + 1) * 3 * f.d_tot + dim;
        q[0] = pc.m;
        q[f.d_tot] = pc.s;
        q[2 * f.d_tot] = pc.w;
        if (tm == 0) {
          float kf[4], sf[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            kf[e] = f.fr_kv[l][e * W + ld];
            sf[e] = f.fr_sc[l][e * W + ld];
          }
          const Part3 pf = half_pool(kf, sf);
          float* q0 = f.part + dim;
          q0[0] = pf.m;
          q0[f.d_tot] = pf.s;
          q0[2 * f.d_tot] = pf.w;
        }
      }
    }
    for (int g = g_lo > 0 ? g_lo : 1; g < g_hi; ++g) {
      float kc[4], sc[4], kq[4], sq[4];
      const f32x4 kc4 = tile4[tile_ix(4 * g, 40 + dd) >> 2], sc4 = tile4[tile_ix(4 * g, 120 + dd) >> 2];
      const f32x4 kq4 = tile4[tile_ix(4 * g, dd) >> 2], sq4 = tile4[tile_ix(4 * g, 80 + dd) >> 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kc[e] = kc4[e];
        sc[e] = sc4[e] + ape_c[e];
        kq[e] = kq4[e];
        sq[e] = sq4[e] + ape_p[e];
      }
      const int64_t jw = j0 + g;
      if (jw < f.n_emit) f.o[jw * f.d_tot + dim] = window_pool(kp, sp, kc, sc);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kp[e] = kq[e];
        sp[e] = sq[e];
      }
    }
    // Group 63's previous half opens the next tile's window 0.
    if (g_hi == 64 && j0 + 64 < f.n_emit) {
      const Part3 pq = half_pool(kp, sp);
      float* q = f.part + ((int64_t)(tm + 1) * 2 + 0) * 3 * f.d_tot + dim;
      q[0] = pq.m;
      q[f.d_tot] = pq.s;
      q[2 * f.d_tot] = pq.w;
    }
  }
  // Kept tokens: call-relative carry_lo .. M-1 that fall in this tile.
  const int64_t s_lo = f.carry_lo > t0 ? f.carry_lo : t0;
  const int64_t s_hi = a.M < t0 + 256 ? a.M : t0 + 256;
  const int n_rows = s_hi > s_lo ? (int)(s_hi - s_lo) : 0;
  for (int item = threadIdx.x; item < n_rows * 160; item += blockDim.x) {
    const int r = item / 160, q = item - r * 160;
    const int run = q / 40, dd = q - run * 40;
    const int dim = tn * 40 + dd;
    if (dim >= f.d_tot) continue;
    const int64_t t = s_lo + r;
    const int l = dim < f.d_attn ? 0 : 1;
    const int ld = dim - (l ? f.d_attn : 0), dl = l ? f.d_idx : f.d_attn, W = f.W[l];
    const int wcol = (run & 1) * dl + ld;  // column within the lane's W-wide block
    float v = tile[tile_ix((int)(t - t0), q)];
    if (run >= 2) v += f.ape[l][(int)(t & 3) * W + wcol];
    const int col = (l ? 2 * f.W[0] : 0) + (run >= 2 ? W : 0) + wcol;
    f.stage[(t - f.carry_lo) * f.n_orig + col] = v;
  }
}

// Eight-wave variant: two waves per SIMD split the K sub-steps of every tile.
// Waves w and w+4 (same SIMD) own the same (BM/WM) x (BN/WN) output block;
// group 0 (waves 0-3) runs K sub-steps 0 and 1 of each 128-byte K tile,
// group 1 sub-steps 2 and 3, both reading the same LDS stage.  While one
// wave of a SIMD waits for LDS data or the barrier, the other issues MFMAs.
// The stage loads (BM + BN rows of 128 bytes, 8 rows per instruction) are
// dealt to the eight waves round-robin.  At the end each group hands half
// of its partial sums to the other through LDS and stores the other half.
template <typename Tin, int BM, int BN, int WM, int WN, bool FUSE>
__global__ void __launch_bounds__(512) proj_splitk_kernel(ProjArgs a, int tiles_m, int tiles_n, int gm) {
  constexpr int kElems = 16 / (int)sizeof(Tin);
  constexpr int BK = 8 * kElems;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 32, FN = TN / 32;
  constexpr int kRows = BM + BN;
  constexpr int kIns = kRows / 8;            // load instructions per stage
  constexpr int kMaxIns = (kIns + 7) / 8;    // per wave
  // 16-byte slots per stage: the operand rows, then one 64-slot pad that
  // takes the spare issue of waves with fewer load instructions.
  constexpr int kStage = kRows * 8 + 64;
  static_assert(WM * WN == 4, "four waves per group");
  static_assert(FM == 2, "the final exchange splits the two 32-row blocks");
  static_assert(kRows % 8 == 0, "whole 8-row loads");
  static_assert(4 * FN * 16 * 64 * 4 <= 3 * kStage * 16, "exchange buffer fits the ring");
  static_assert(3 * kStage * 16 <= 160 * 1024, "ring fits the LDS");
  static_assert(!FUSE || (BM == 256 && BN == 160), "the fused epilogue holds a 256 x 160 tile");
  static_assert(!FUSE || 2 * 4 * FN * 16 * 64 <= BM * BN, "both groups' parked partial sums fit the tile");
  // The fused epilogue stages the whole fp32 tile (160 KiB) in LDS.
  constexpr int kSmem = FUSE && BM * BN / 4 > 3 * kStage ? BM * BN / 4 : 3 * kStage;
  static_assert(kSmem >= 3 * kStage, "ring fits");
  __shared__ u32x4 smem[kSmem];

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

  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int grp = wave >> 2, wq = wave & 3;
  const int h = lane >> 5, r32 = lane & 31;

  // Stage row r < BM is x row m0 + r, row BM + c is weight row n0 + c.
  // Loads go through buffer descriptors with per-lane byte offsets; the K
  // tile advances through the scalar offset.  Waves without an i-th
  // instruction issue an empty load into the stage's pad instead.
  constexpr int kElemBytes = (int)sizeof(Tin);
  const int64_t rows_left = a.M - m0;
  const char* x_base = reinterpret_cast<const char*>(a.x) + m0 * a.K * kElemBytes;
  const int x_bytes = (int)((rows_left < BM ? rows_left : BM) * a.K * kElemBytes);
  const void* l_base[kMaxIns];
  int l_bytes[kMaxIns];
  uint32_t l_off[kMaxIns];
  int l_slot[kMaxIns];
#pragma unroll
  for (int i = 0; i < kMaxIns; ++i) {
    const int ins = min(wave + 8 * i, kIns - 1);
    l_slot[i] = ins * 64;
    const int row0 = ins * 8;  // uniform first row of the instruction
    const int row = row0 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    if (row0 < BM) {
      const int r = row < rows_left ? row : (int)rows_left - 1;
      l_base[i] = x_base;
      l_bytes[i] = x_bytes;
      l_off[i] = (uint32_t)((r * a.K + chunk * kElems) * kElemBytes);
    } else if constexpr (FUSE) {
      // Tile column q: run q / 40 (kv prev, kv cur, score prev, score cur)
      // of dim 40*tn + q % 40.  Runs, lanes and the padding past d_tot all
      // start at multiples of 8, so an instruction's 8 rows are 8
      // consecutive rows of one weight matrix (padding re-reads real rows).
      const FuseArgs& f = a.fuse;
      const int q0 = row0 - BM;
      const int run = q0 / 40;
      int dim0 = tn * 40 + q0 % 40;
      dim0 = dim0 < f.d_tot ? dim0 : f.d_tot - 8;
      const int l = dim0 < f.d_attn ? 0 : 1;
      const int dl = l ? f.d_idx : f.d_attn;
      const int wrow = dim0 - (l ? f.d_attn : 0) + (run & 1) * dl + (lane >> 3);
      const int si = 2 * l + (run >> 1);
      const void* w = a.seg[0].w;
      int cn = a.seg[0].n;
      if (si == 1) { w = a.seg[1].w; cn = a.seg[1].n; }
      if (si == 2) { w = a.seg[2].w; cn = a.seg[2].n; }
      if (si == 3) { w = a.seg[3].w; cn = a.seg[3].n; }
      l_base[i] = w;
      l_bytes[i] = cn * a.K * kElemBytes;
      l_off[i] = (uint32_t)((wrow * a.K + chunk * kElems) * kElemBytes);
    } else {
      int n_first = n0 + row0 - BM;
      n_first = n_first < a.N ? n_first : a.N - 1;
      int n = n0 + row - BM;
      n = n < a.N ? n : a.N - 1;
      const void* w = a.seg[0].w;
      int c0 = a.seg[0].col0, cn = a.seg[0].n;
      if (a.n_seg > 1 && n_first >= a.seg[1].col0) { w = a.seg[1].w; c0 = a.seg[1].col0; cn = a.seg[1].n; }
      if (a.n_seg > 2 && n_first >= a.seg[2].col0) { w = a.seg[2].w; c0 = a.seg[2].col0; cn = a.seg[2].n; }
      if (a.n_seg > 3 && n_first >= a.seg[3].col0) { w = a.seg[3].w; c0 = a.seg[3].col0; cn = a.seg[3].n; }
      l_base[i] = w;
      l_bytes[i] = cn * a.K * kElemBytes;
      l_off[i] = (uint32_t)(((n - c0) * a.K + chunk * kElems) * kElemBytes);
    }
    if (wave + 8 * i >= kIns) {
      // Spare issue of a wave with fewer instructions: an empty buffer range
      // (every lane out of range, nothing fetched) into the stage's pad.
      l_slot[i] = kRows * 8;
      l_bytes[i] = 0;
      l_off[i] = 0;
    }
  }
  // Each XCD starts its K walk at its own eighth of K (as in the ratio-128
  // kernel below): cold weights are fetched from HBM by one XCD at a time.
  const int nk_all4 = a.K / BK;
  const int rot4 = __builtin_amdgcn_readfirstlane((x * nk_all4) / kXcds);
  auto issue_one = [&](int kt, int st, int i) {
    int kr = kt + rot4; if (kr >= nk_all4) kr -= nk_all4;
    const uint32_t k0b = (uint32_t)(kr * BK * kElemBytes);
    __attribute__((address_space(3))) u32x4* base =
        (__attribute__((address_space(3))) u32x4*)(smem + st * kStage);
    load_lds16(l_base[i], l_bytes[i], (__attribute__((address_space(3))) void*)(base + l_slot[i]), l_off[i], k0b);
  };
  auto issue = [&](int kt, int st) {
#pragma unroll
    for (int i = 0; i < kMaxIns; ++i) issue_one(kt, st, i);
  };

  const int wm = wq / WN, wn = wq % WN;
  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x16{};

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
      const int row = BM + wn * TN + fn * 32 + r32;
      fb[fn] = base[row * 8 + (c ^ swz(row))];
    }
  };
  // Fragment f (x blocks, then weight blocks) of K sub-step kk of stage st.
  auto frag = [&](u32x4 (&fa)[FM], u32x4 (&fb)[FN], int f, int st, int kk) {
    const u32x4* base = smem + st * kStage;
    const int c = 2 * kk + h;
    if (f < FM) {
      const int row = wm * TM + f * 32 + r32;
      fa[f] = base[row * 8 + (c ^ swz(row))];
    } else {
      const int row = BM + wn * TN + (f - FM) * 32 + r32;
      fb[f - FM] = base[row * 8 + (c ^ swz(row))];
    }
  };
  // One K sub-step in a fixed issue order: MFMA i, then fragment i of the
  // next sub-step, then (spread evenly) one of the nd loads of tile kt_load.
  auto sub_step = [&](const u32x4 (&ca)[FM], const u32x4 (&cb)[FN], u32x4 (&na)[FM], u32x4 (&nb)[FN], int st_next,
                      int kk_next, int kt_load, int st_load, int nd) {
    constexpr int kM = FM * FN, kR = FM + FN;
    int d = 0;
#pragma unroll
    for (int i = 0; i < kM; ++i) {
      mfma_chunk<Tin>(ca[i / FN], cb[i % FN], acc[i / FN][i % FN]);
      if (i < kR) frag(na, nb, i, st_next, kk_next);
      if (nd > 0 && (i * nd) / kM != ((i + 1) * nd) / kM) {
        issue_one(kt_load, st_load, d);
        ++d;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    // Fewer MFMAs than fragments or loads: issue the rest.
#pragma unroll
    for (int f = kM; f < kR; ++f) frag(na, nb, f, st_next, kk_next);
    for (; d < nd; ++d) issue_one(kt_load, st_load, d);
  };
  const int nk = a.K / BK;
  const int kk0 = 2 * grp;
  issue(0, 0);
  issue(min(1, nk - 1), 1);
  issue(min(2, nk - 1), 2);
  wait_vm<2 * kMaxIns>();  // tile 0 (loads complete in issue order)
  asm volatile("s_barrier" ::: "memory");
  frags(fa0, fb0, 0, kk0);
  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % 3;
    sub_step(fa0, fb0, fa1, fb1, st, kk0 + 1, 0, 0, 0);
    // Past the barrier tile kt+1 has landed for every wave (only this wave's
    // kMaxIns loads of tile kt+2 may still be in flight) and every wave's
    // reads of stage st have completed, so the loads below refill stage st
    // with tile kt+3, two iterations ahead of its use.  Past the last tile
    // they re-read the last tile into a stage nothing reads again, so the
    // loop body has no branches and the compiler's wait counts stay exact.
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lds<kMaxIns>();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    sub_step(fa1, fb1, fa0, fb0, (kt + 1) % 3, kk0, min(kt + 3, nk - 1), st, kMaxIns);
  }
  wait_vm<0>();  // the exchange below reuses the ring

  if constexpr (FUSE) {
    fused_r4_epilogue<WM>(a, acc, reinterpret_cast<float*>(smem), tm, tn, wq, grp, lane);
    return;
  }

  // Exchange: round r, group 1-r parks its partial sums of block fm = r in
  // LDS (lane-major, conflict free) and group r adds them; group r then
  // owns block r.
  asm volatile("s_barrier" ::: "memory");
  float* red = reinterpret_cast<float*>(smem);
#pragma unroll
  for (int r = 0; r < 2; ++r) {
    if (grp != r) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) red[((wq * FN + fn) * 16 + v) * 64 + lane] = acc[r][fn][v];
    }
    __syncthreads();
    if (grp == r) {
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[r][fn][v] += red[((wq * FN + fn) * 16 + v) * 64 + lane];
    }
    __syncthreads();
  }

  // 32x32 accumulator layout: lane holds column r32, rows 8*(v/4) + 4*h + v%4.
#pragma unroll
  for (int fm = 0; fm < FM; ++fm) {
    if (fm != grp) continue;
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

// K-split projection: plane 0 += planes 1 .. n_split-1, added in order, so
// the sum is the same on every run.
__global__ void __launch_bounds__(256) proj_sum_planes_kernel(float4* out, int64_t n4, int n_split, int64_t stride4) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n4; i += (int64_t)gridDim.x * 256) {
    float4 v = out[i];
    for (int s = 1; s < n_split; ++s) {
      const float4 w = out[i + s * stride4];
      v.x += w.x;
      v.y += w.y;
      v.z += w.z;
      v.w += w.w;
    }
    out[i] = v;
  }
}

// ---------------------------------------------------------------------------
// proj_r128_splitk4_kernel: the fused ratio-128 projection (128 x 128 tiles,
// one window per tile) on eight waves, two per SIMD.  Wave w = 2s + n owns
// the 128 x 64 output block n (4 x 2 accumulators) and runs K sub-step s of
// every 64-column K tile, a four-way split of K: per MFMA it reads 0.75 KiB
// of fragments, against 1 KiB for a 64 x 64 block, and two waves per SIMD
// keep the LDS busy.  Stages are 128-byte rows in a 4-stage ring; after the
// barrier of iteration j stage j % 4 is free and is refilled with tile j + 4.
// The partial sums meet in two fixed rounds, ((s0 + s2) + (s1 + s3)).
// ---------------------------------------------------------------------------
template <typename Tin>
__global__ void __launch_bounds__(512) proj_r128_splitk4_kernel(ProjArgs a, int tiles_m, int tiles_n, int gm) {
  constexpr int BM = 128, BN = 128, kNst = 4;
  constexpr int kElems = 16 / (int)sizeof(Tin);
  constexpr int kElemBytes = (int)sizeof(Tin);
  constexpr int BK = 8 * kElems;
  constexpr int FM = 4, FN = 2;
  constexpr int kRows = BM + BN;
  constexpr int kIns = kRows / 8;          // 8-row load instructions per stage
  constexpr int kMaxIns = kIns / 8;        // per wave
  constexpr int kStage = kRows * 8;        // 16-byte slots per stage
  static_assert(kIns % 8 == 0, "every wave issues the same loads");
  static_assert(kNst * kStage * 16 <= 160 * 1024, "ring fits the LDS");
  static_assert(4 * 8192 * 4 <= kNst * kStage * 16, "parked partial sums fit the ring");
  __shared__ u32x4 smem[kNst * kStage];

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

  const int wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
  const int ks = wave >> 1, wn = wave & 1;
  const int h = lane >> 5, r32 = lane & 31;

  // Stage row r < BM is x row m0 + r; row BM + q is weight row 64*tn + q%64
  // of wkv (q < 64) or wgate.  Instruction i of this wave covers rows
  // 8*(wave + 8i) .. +7; the K tile advances through the scalar offset.
  const int64_t rows_left = a.M - m0;
  const char* x_base = reinterpret_cast<const char*>(a.x) + m0 * a.K * kElemBytes;
  const int x_bytes = (int)((rows_left < BM ? rows_left : BM) * a.K * kElemBytes);
  const void* l_base[kMaxIns];
  int l_bytes[kMaxIns];
  uint32_t l_off[kMaxIns];
  int l_slot[kMaxIns];
#pragma unroll
  for (int i = 0; i < kMaxIns; ++i) {
    const int ins = wave + 8 * i;
    l_slot[i] = ins * 64;
    const int row0 = ins * 8;
    const int row = row0 + (lane >> 3);
    const int chunk = (lane & 7) ^ swz(row);
    if (row0 < BM) {
      const int r = row < rows_left ? row : (int)rows_left - 1;
      l_base[i] = x_base;
      l_bytes[i] = x_bytes;
      l_off[i] = (uint32_t)((r * a.K + chunk * kElems) * kElemBytes);
    } else {
      const int q0 = row0 - BM;
      const int wrow = tn * 64 + (q0 & 63) + (lane >> 3);
      l_base[i] = q0 < 64 ? a.seg[0].w : a.seg[1].w;
      l_bytes[i] = a.seg[0].n * a.K * kElemBytes;
      l_off[i] = (uint32_t)((wrow * a.K + chunk * kElems) * kElemBytes);
    }
  }
  // Each XCD starts its K walk at its own eighth of K (tile kt reads K tile
  // (kt + rot) mod nk).  The workgroups of one XCD stay in step, sharing its
  // L2; different XCDs read different weight lines at any moment, so cold
  // weights come from HBM once and the other XCDs find them in the Infinity
  // Cache (long stack, weights cold: prefill 30.6 -> 29.6 ms per step).
  const int nk_all = a.K / BK;
  const int rot = __builtin_amdgcn_readfirstlane((x * nk_all) / kXcds);
  auto issue = [&](int kt, int st) {
    int kr = kt + rot; if (kr >= nk_all) kr -= nk_all;
    const uint32_t k0b = (uint32_t)(kr * BK * kElemBytes);
    __attribute__((address_space(3))) u32x4* base = (__attribute__((address_space(3))) u32x4*)(smem + st * kStage);
#pragma unroll
    for (int i = 0; i < kMaxIns; ++i)
      load_lds16(l_base[i], l_bytes[i], (__attribute__((address_space(3))) void*)(base + l_slot[i]), l_off[i], k0b);
  };
  auto issue_one = [&](int kt, int st, int i) {
    int kr = kt + rot; if (kr >= nk_all) kr -= nk_all;
    const uint32_t k0b = (uint32_t)(kr * BK * kElemBytes);
    __attribute__((address_space(3))) u32x4* base = (__attribute__((address_space(3))) u32x4*)(smem + st * kStage);
    load_lds16(l_base[i], l_bytes[i], (__attribute__((address_space(3))) void*)(base + l_slot[i]), l_off[i], k0b);
  };

  f32x16 acc[FM][FN];
#pragma unroll
  for (int fm = 0; fm < FM; ++fm)
#pragma unroll
    for (int fn = 0; fn < FN; ++fn) acc[fm][fn] = f32x16{};
  // Fragment f (x blocks, then weight blocks) of this wave's sub-step of stage st.
  const int c = 2 * ks + h;
  auto frag = [&](u32x4 (&fa)[FM], u32x4 (&fb)[FN], int f, int st) {
    const u32x4* base = smem + st * kStage;
    if (f < FM) {
      const int row = f * 32 + r32;
      fa[f] = base[row * 8 + (c ^ swz(row))];
    } else {
      const int row = BM + wn * 64 + (f - FM) * 32 + r32;
      fb[f - FM] = base[row * 8 + (c ^ swz(row))];
    }
  };
  // One tile: MFMA i, then fragment i of the next tile, then (spread
  // evenly) the loads of tile kt_load into stage st_load.
  auto step = [&](const u32x4 (&ca)[FM], const u32x4 (&cb)[FN], u32x4 (&na)[FM], u32x4 (&nb)[FN], int st_next,
                  int kt_load, int st_load) {
    constexpr int kM = FM * FN, kR = FM + FN;
    int d = 0;
#pragma unroll
    for (int i = 0; i < kM; ++i) {
      mfma_chunk<Tin>(ca[i / FN], cb[i % FN], acc[i / FN][i % FN]);
      if (i < kR) frag(na, nb, i, st_next);
      if ((i * kMaxIns) / kM != ((i + 1) * kMaxIns) / kM) {
        issue_one(kt_load, st_load, d);
        ++d;
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  u32x4 fa0[FM], fb0[FN], fa1[FM], fb1[FN];
  const int nk = a.K / BK;
#pragma unroll
  for (int s = 0; s < kNst; ++s) issue(min(s, nk - 1), s);
  wait_vm<(kNst - 1) * kMaxIns>();  // tile 0 (loads complete in issue order)
  asm volatile("s_barrier" ::: "memory");
#pragma unroll
  for (int f = 0; f < FM + FN; ++f) frag(fa0, fb0, f, 0);
  // Past the barrier of tile kt, tile kt+1 has landed for every wave (this
  // wave's loads of tiles kt+2 and kt+3 may still be in flight) and every
  // wave's reads of stage kt % 4 have completed, so the step refills it with
  // tile kt+4.  Past the last tile the loads re-read the last tile into a
  // stage nothing reads again, so the loop body has no branches.
  auto tile_step = [&](const u32x4 (&ca)[FM], const u32x4 (&cb)[FN], u32x4 (&na)[FM], u32x4 (&nb)[FN], int kt) {
    __builtin_amdgcn_sched_barrier(0);
    wait_vm_lds<(kNst - 2) * kMaxIns>();
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
    step(ca, cb, na, nb, (kt + 1) % kNst, min(kt + kNst, nk - 1), kt % kNst);
  };
  int kt = 0;
  for (; kt + 1 < nk; kt += 2) {
    tile_step(fa0, fb0, fa1, fb1, kt);
    tile_step(fa1, fb1, fa0, fb0, kt + 1);
  }
  if (kt < nk) tile_step(fa0, fb0, fa1, fb1, kt);  // odd number of K tiles
  wait_vm<0>();  // the epilogue reuses the ring

  // Epilogue (Part 3 §4): the tile is window j = tm of a call that starts
  // on a window boundary.  APE values first, so that their latency hides
  // behind the combine.
  const FuseArgs& f = a.fuse;
  const int D = f.d_attn;
  const int64_t t0 = m0;
  const int64_t jw = tm;
  const int dd = t >> 3, qq = t & 7;
  const int dim = tn * 64 + dd;
  float ape[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) ape[e] = f.ape[0][(qq * 16 + e) * D + dim];
  float* tile = reinterpret_cast<float*>(smem);
  f32x4* tile4 = reinterpret_cast<f32x4*>(smem);
  // Partial sums park in 16-byte chunks (four consecutive v), lane-major.
  constexpr int kPark4 = FM * FN * 4 * 64;  // chunks of one wave's partial sums
  asm volatile("s_barrier" ::: "memory");  // every wave is done with the ring
  auto park = [&](int slot) {
#pragma unroll
    for (int i = 0; i < FM * FN; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x16& s = acc[i / FN][i % FN];
        tile4[slot * kPark4 + (i * 4 + j) * 64 + lane] = f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
      }
  };
  auto add = [&](int slot) {
#pragma unroll
    for (int i = 0; i < FM * FN; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4 p = tile4[slot * kPark4 + (i * 4 + j) * 64 + lane];
        f32x16& s = acc[i / FN][i % FN];
        s[4 * j] += p.x;
        s[4 * j + 1] += p.y;
        s[4 * j + 2] += p.z;
        s[4 * j + 3] += p.w;
      }
  };
  // Round 1: splits 2 and 3 park, splits 0 and 1 add them.
  if (ks >= 2) park((ks - 2) * 2 + wn);
  __syncthreads();
  if (ks < 2) add(ks * 2 + wn);
  __syncthreads();
  // Round 2: split 1 parks, split 0 adds.
  if (ks == 1) park(wn);
  __syncthreads();
  if (ks == 0) add(wn);
  __syncthreads();
  // 32x32 accumulator layout: lane holds column r32, rows 8*(v/4) + 4*h + v%4;
  // rows 8j + 4h .. 8j + 4h + 3 are one 4-row group.
  if (ks == 0) {
#pragma unroll
    for (int fm = 0; fm < FM; ++fm)
#pragma unroll
      for (int fn = 0; fn < FN; ++fn)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const f32x16& s = acc[fm][fn];
          tile4[tile128_ix(fm * 32 + 8 * j + 4 * h, wn * 64 + fn * 32 + r32) >> 2] =
              f32x4{s[4 * j], s[4 * j + 1], s[4 * j + 2], s[4 * j + 3]};
        }
  }
  __syncthreads();
  // Eight lanes per dim pool 16 tokens each and merge by shuffles.
  if (jw < f.n_emit) {
    float kv[16], sc[16];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const f32x4 k4 = tile4[tile128_ix(qq * 16 + 4 * i, dd) >> 2];
      const f32x4 s4 = tile4[tile128_ix(qq * 16 + 4 * i, 64 + dd) >> 2];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        kv[4 * i + e] = k4[e];
        sc[4 * i + e] = s4[e] + ape[4 * i + e];
      }
    }
    float m = sc[0];
#pragma unroll
    for (int e = 1; e < 16; ++e) m = fmaxf(m, sc[e]);
    const float ms = m == -INFINITY ? 0.f : m;
    float s = 0.f, w = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float xw = pool_exp(sc[e] - ms);
      s += xw;
      w = fmaf(xw, kv[e], w);
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) {
      const float m2 = lane_xor(m, o), s2 = lane_xor(s, o), w2 = lane_xor(w, o);
      const float mm = fmaxf(m, m2);
      const float mms = mm == -INFINITY ? 0.f : mm;
      const float f1 = pool_exp(m - mms), f2 = pool_exp(m2 - mms);
      s = fmaf(s, f1, s2 * f2);
      w = fmaf(w, f1, w2 * f2);
      m = mm;
    }
    if (qq == 0) f.o[jw * D + dim] = s > 0.f ? w / s : 0.f;
  }
  // Kept tokens: call-relative carry_lo .. M-1 that fall in this tile.
  const int64_t s_lo = f.carry_lo > t0 ? f.carry_lo : t0;
  const int64_t s_hi = a.M < t0 + 128 ? a.M : t0 + 128;
  const int n_rows = s_hi > s_lo ? (int)(s_hi - s_lo) : 0;
  for (int item = t; item < n_rows * 128; item += 512) {
    const int r = item >> 7, qc = item & 127;
    const int64_t tok = s_lo + r;
    const int d = tn * 64 + (qc & 63);
    float v = tile[tile128_ix((int)(tok - t0), qc)];
    if (qc >= 64) v += f.ape[0][(int)(tok & 127) * D + d];
    f.stage[(tok - f.carry_lo) * f.n_orig + (qc >= 64 ? D : 0) + d] = v;
  }
}

template <typename Tin>
void launch_cfg(const ProjArgs& a, TileCfg c, hipStream_t stream, const Timing& tm) {
  const int tiles_m = (int)((a.M + c.bm - 1) / c.bm);
  const int tiles_n = (a.N + c.bn - 1) / c.bn;
  const dim3 grid((unsigned)(tiles_m * tiles_n), (unsigned)a.k_split);
  const int gm = 4;
  if (c.bm == 256)  // no K split on this kernel (the planner never asks for one)
    hipExtLaunchKernelGGL((proj_splitk_kernel<Tin, 256, 160, 4, 1, false>), dim3(grid.x), dim3(512), 0, stream, tm.start,
                          tm.stop, 0, a, tiles_m, tiles_n, gm);
  else if (c.bm == 128)
    hipExtLaunchKernelGGL((proj_mfma_kernel<Tin, 128, 128, 2, 2>), grid, dim3(kThreads), 0, stream, tm.start, tm.stop, 0, a, tiles_m,
                       tiles_n, gm);
  else
    hipExtLaunchKernelGGL((proj_mfma_kernel<Tin, 64, 64, 2, 2>), grid, dim3(kThreads), 0, stream, tm.start, tm.stop, 0, a, tiles_m,
                       tiles_n, gm);
}

}  // namespace

namespace {

// Measured time of one tile per CU over K = 4096 on one MI355X, in
// microseconds: 256 x 160, 128 x 128 and 64 x 64.  Two 64 x 64 tiles share a
// CU at once; each further tile per CU adds kExtra64 of a round.  Only the
// ratios matter for the choices below.
constexpr double kRoundUs256 = 75.0, kRoundUs128 = 42.0, kRoundUs64 = 25.0, kExtra64 = 0.7;
// Fused grids below these sizes leave enough CUs idle that the plain, K-split
// projection plus a pool pass over its output is as fast or faster (measured
// break-even on hidden 4096: ratio 4 between 1024 and 1280 tokens, 80
// workgroups of 256 x 160; ratio 128 at about 512 tokens, 32 workgroups).
constexpr int64_t kMinFusedGrid4 = 80, kMinFusedGrid128 = 32;

int tile_cols(int bm) { return bm == 256 ? 160 : bm; }
int64_t tile_slots(int bm) { return bm == 64 ? 512 : 256; }
double round_us(int bm) { return bm == 256 ? kRoundUs256 : bm == 128 ? kRoundUs128 : kRoundUs64; }

// K ranges for a plain projection with `tiles` output tiles: the largest
// power of two (at most 16) that keeps every split resident in one round,
// k_split * M <= kSplitRows, and whole 64-column K ranges of at least 128.
int split_for(int bm, int64_t tiles, int64_t M, int K) {
  int s = 1;
  if (bm == 256) return s;  // the 256 x 160 kernel has no K split
  while (s < 16) {
    const int s2 = 2 * s;
    if (tiles * s2 > tile_slots(bm) || M * s2 > kSplitRows || K % (64 * s2) != 0 || K / s2 < 128) break;
    s = s2;
  }
  return s;
}

double plan_us(int bm, int64_t M, int N, int K, int* k_split) {
  const int64_t tiles = ((M + bm - 1) / bm) * ((N + tile_cols(bm) - 1) / tile_cols(bm));
  const int s = split_for(bm, tiles, M, K);
  if (k_split) *k_split = s;
  const int64_t per_cu = (tiles * s + 255) / 256;
  const double rounds = bm == 64 ? 1.0 + kExtra64 * (double)(per_cu - 1) : (double)per_cu;
  return rounds * round_us(bm) * ((double)K / s / 4096.0);
}

}  // namespace

// Plain projection plan: the tile shape with the least estimated time,
// ties to the larger tile (fewer K-tile reloads).
ProjPlan proj_plan(int64_t M, int N, int K) {
  ProjPlan best{256, 1};
  double best_us = -1.0;
  for (int bm : {256, 128, 64}) {
    int s = 1;
    const double us = plan_us(bm, M, N, K, &s);
    if (best_us < 0.0 || us < best_us) {
      best_us = us;
      best = ProjPlan{bm, s};
    }
  }
  return best;
}

bool use_fused_projection(int ratio, int64_t M, int N, int K, int d_tot) {
  (void)N;
  const int64_t grid_f = ratio == 4 ? ((M + 255) / 256) * ((d_tot + 39) / 40) : ((M + 127) / 128) * (d_tot / 64);
  const int64_t tile_f = ratio == 4 ? 256 * 160 : 128 * 128;
  // Short either way (small hidden sizes): keep the fused path.
  if (((grid_f + 255) / 256) * tile_f * K < int64_t(256 * 160) * 1024) return true;
  return grid_f >= (ratio == 4 ? kMinFusedGrid4 : kMinFusedGrid128);
}

hipError_t launch_proj(const ProjArgs& a, int in_dtype, hipStream_t stream, const Timing& tm) {
  if (a.fuse.on && a.fuse.ratio == 128) {
    const int tiles_m = (int)((a.M + 127) / 128);
    const int tiles_n = a.fuse.d_attn / 64;
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    if (in_dtype == 1)
      hipExtLaunchKernelGGL((proj_r128_splitk4_kernel<uint16_t>), grid, dim3(512), 0, stream, tm.start, tm.stop, 0, a,
                            tiles_m, tiles_n, 4);
    else
      hipExtLaunchKernelGGL((proj_r128_splitk4_kernel<float>), grid, dim3(512), 0, stream, tm.start, tm.stop, 0, a,
                            tiles_m, tiles_n, 4);
    return hipGetLastError();
  }
  if (a.fuse.on) {
    const int tiles_m = (int)((a.M + 255) / 256);
    const int tiles_n = (a.fuse.d_tot + 39) / 40;
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    if (in_dtype == 1)
      hipExtLaunchKernelGGL((proj_splitk_kernel<uint16_t, 256, 160, 4, 1, true>), grid, dim3(512), 0, stream, tm.start,
                            tm.stop, 0, a, tiles_m, tiles_n, 4);
    else
      hipExtLaunchKernelGGL((proj_splitk_kernel<float, 256, 160, 4, 1, true>), grid, dim3(512), 0, stream, tm.start,
                            tm.stop, 0, a, tiles_m, tiles_n, 4);
    return hipGetLastError();
  }
  const ProjPlan pl = proj_plan(a.M, a.N, a.K);
  if (pl.k_split != a.k_split || (int64_t)a.k_len * a.k_split != a.K || a.split_stride != a.M * a.N)
    return hipErrorInvalidValue;
  const TileCfg c = pl.bm == 256 ? TileCfg{256, 160} : pl.bm == 128 ? TileCfg{128, 128} : TileCfg{64, 64};
  const Timing t_gemm{tm.start, a.k_split > 1 ? nullptr : tm.stop};
  if (in_dtype == 1)
    launch_cfg<uint16_t>(a, c, stream, t_gemm);
  else
    launch_cfg<float>(a, c, stream, t_gemm);
  if (a.k_split > 1) {
    const int64_t n4 = a.M * a.N / 4;
    const int64_t g = (n4 + 255) / 256;
    hipExtLaunchKernelGGL(proj_sum_planes_kernel, dim3((unsigned)(g < 1024 ? g : 1024)), dim3(256), 0, stream, nullptr,
                          tm.stop, 0, reinterpret_cast<float4*>(a.out), n4, a.k_split, a.split_stride / 4);
  }
  return hipGetLastError();
}

}  // namespace ds4c
