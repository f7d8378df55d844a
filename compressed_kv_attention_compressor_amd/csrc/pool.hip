// Compressor pool kernels: APE add, window gather (projection workspace or
// carried frontier), per-dimension softmax pool, RMS norm, tail RoPE,
// FP8 / Hadamard+FP4 round trip, row append and frontier carry.
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
// Only the first one or two windows of a call can touch such tokens.
//
// Ratio 4 runs in two launches: one window per workgroup, then a wide copy
// that carries the frontier.  Ratio 128 runs in two: a wide partial-pool
// launch with no cross-workgroup dependency, then a finishing launch that
// merges the partials, normalises, rotates and quantises each row while
// extra workgroups carry the frontier.  In both, a launch boundary orders the
// carry after every read of the incoming frontier.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace ds4c {

namespace {

// DPL dims of token p, starting at column c of the lane's W-wide kv / score
// blocks (score with APE added).
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
    load_vec<DPL>(kv, L.fr_kv + row * L.W + c);
    load_vec<DPL>(sc, L.fr_sc + row * L.W + c);
    return;
  }
  const float* src = a.proj + (p - a.n0) * a.ld;
  load_vec_stream<DPL>(kv, src + L.kv_col + c);
  load_vec_stream<DPL>(sc, src + L.sc_col + c);
  float ape[DPL];
  load_vec<DPL>(ape, L.ape + pr * L.W + c);
#pragma unroll
  for (int i = 0; i < DPL; ++i) sc[i] += ape[i];
}

// Pooled dims c .. c+DPL-1 of ratio-4 window k of one lane.
template <int DPL>
__device__ __forceinline__ void r4_pool(const PoolArgs& a, const LaneDev& L, int64_t k, int c, float (&o)[DPL]) {
  float kv[8][DPL], sc[8][DPL];
#pragma unroll
  for (int e = 0; e < 8; ++e) fetch_token<4, DPL>(a, L, 4 * k - 4 + e, (e < 4 ? 0 : L.D) + c, kv[e], sc[e]);
  pool_entries<8, DPL>(kv, sc, o);
}

// Frontier carry after a call, by one whole workgroup.  With n = n0 + T,
// c = n % ratio, m = n - c: ratio 4 keeps tokens m-4 .. m-1 in rows 0..3 and
// m .. n-1 in rows 4 .. 3+c; ratio 128 keeps m .. n-1 in rows 0 .. c-1.  Only
// rows that change are written.  Every read of the incoming frontier by this
// call's windows has completed before this runs.
template <int R>
__device__ void carry_frontier(const PoolArgs& a) {
  const int64_t n = a.n0 + a.T;
  const int64_t m = n - (n & (R - 1));
  const int c4 = threadIdx.x * 4, step = 4 * blockDim.x;
  if (R == 4) {
    const int64_t m0 = a.n0 - (a.n0 & 3);
    // Old tokens that move from the current half to the previous half.
    if (m > m0 && m - 4 < a.n0) {
      for (int l = 0; l < a.n_lanes; ++l) {
        const LaneDev& L = a.lane[l];
        for (int64_t p = m - 4; p < a.n0; ++p) {
          const int src = 4 + (int)(p & 3), dst = (int)(p & 3);
          for (int c = c4; c < L.W; c += step) {
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
      for (int c = c4; c < L.W; c += step) {
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

// The frontier carry spread over n_groups workgroups: kept token p's kv and
// score (APE added) go from the projection workspace to row p - (m - 4)
// (ratio 4) or p - m (ratio 128), one float4 per thread and step.  A short
// ratio-4 call that also moves old tokens within the frontier (rows 4.. ->
// 0..3) runs carry_frontier on workgroup 0 alone, because its new tokens may
// overwrite rows the move reads.  W / 4 is a power of two, so items decode
// by shifts.
template <int R>
__device__ void carry_frontier_wide(const PoolArgs& a, int group, int n_groups) {
  const int64_t n = a.n0 + a.T;
  const int64_t m = n - (n & (R - 1));
  if (R == 4 && m > a.n0 - (a.n0 & 3) && m - 4 < a.n0) {
    if (group == 0) carry_frontier<R>(a);
    return;
  }
  const int64_t first = R == 4 ? (m - 4 > a.n0 ? m - 4 : a.n0) : (m > a.n0 ? m : a.n0);
  const int row0 = R == 4 ? (int)(first - (m - 4)) : (int)(first - m);
  const int pr0 = (int)(first & (R - 1));
  const float* src0 = a.proj + (first - a.n0) * a.ld;
  const int gid = group * (int)blockDim.x + (int)threadIdx.x, stride = n_groups * (int)blockDim.x;
  for (int l = 0; l < a.n_lanes; ++l) {
    const LaneDev& L = a.lane[l];
    const int sh = __builtin_ctz(L.W / 4), mask = L.W / 4 - 1;
    const int count = (int)(n - first) * 2 << sh;
    for (int i = gid; i < count; i += stride) {
      const int tk = i >> sh, j = tk >> 1, c = (i & mask) * 4;
      float4 v = *reinterpret_cast<const float4*>(src0 + (int64_t)j * a.ld + ((tk & 1) ? L.sc_col : L.kv_col) + c);
      if (tk & 1) {
        const float4 ap = *reinterpret_cast<const float4*>(L.ape + ((pr0 + j) & (R - 1)) * L.W + c);
        v.x += ap.x; v.y += ap.y; v.z += ap.z; v.w += ap.w;
      }
      *reinterpret_cast<float4*>(((tk & 1) ? L.fr_sc : L.fr_kv) + (row0 + j) * L.W + c) = v;
    }
  }
}

// Workgroups for the wide carry: one float4 per thread (256 threads per
// workgroup), at most 64 workgroups.
int carry_groups(const PoolArgs& a) {
  const int64_t n = a.n0 + a.T, R = a.ratio;
  const int64_t m = n - n % R;
  const int64_t first = R == 4 ? (m - 4 > a.n0 ? m - 4 : a.n0) : (m > a.n0 ? m : a.n0);
  int64_t items = 0;
  for (int l = 0; l < a.n_lanes; ++l) items += (n - first) * 2 * (a.lane[l].W / 4);
  const int64_t g = (items + 255) / 256;
  return (int)(g < 1 ? 1 : g > 64 ? 64 : g);
}

// One ratio-4 window on one workgroup: SA attention waves (D_attn/SA dims
// each, DPLA per lane) and one indexer wave (the whole indexer row, DPLI per
// lane).  The attention row's sum of squares is reduced through LDS.
template <int SA, int DPLA, int DPLI>
__device__ __forceinline__ void r4_window(const PoolArgs& a, int64_t k, float* s_ss) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  if (wave < SA) {
    const LaneDev& L = a.lane[0];
    const int d0 = wave * (kWave * DPLA) + lane * DPLA;
    float nw[DPLA], o[DPLA];
    load_vec<DPLA>(nw, L.norm_w + d0);
    r4_pool<DPLA>(a, L, k, d0, o);
    const float ss = wave_sum(row_sumsq<DPLA>(o));
    if (lane == 0) s_ss[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int s = 0; s < SA; ++s) tot += s_ss[s];
    float* pre = L.prequant ? L.prequant + (k - a.k_lo) * L.D : nullptr;
    const RowConsts<DPLA> rc = row_consts<DPLA>(d0, L.D, a.n_rot, a.log2_base, k, 4);
    finish_row_part<DPLA>(o, nw, L, rms_inv(tot, L.D, a.rms_eps), d0, a.n_rot, rc, pre, L.rows + k * L.D, lane);
  } else {
    const LaneDev& L = a.lane[1];
    float nw[DPLI], o[DPLI];
    load_vec<DPLI>(nw, L.norm_w + lane * DPLI);
    r4_pool<DPLI>(a, L, k, lane * DPLI, o);
    __syncthreads();
    float* pre = L.prequant ? L.prequant + (k - a.k_lo) * L.D : nullptr;
    const RowConsts<DPLI> rc = row_consts<DPLI>(lane * DPLI, L.D, a.n_rot, a.log2_base, k, 4);
    finish_row_wave<DPLI>(o, nw, L, a.n_rot, a.rms_eps, rc, pre, L.rows + k * L.D, lane);
  }
  __syncthreads();
}

// Ratio 4: one window per workgroup, window k_lo + b on workgroup b.  The
// leading windows read the incoming frontier; the carry that rewrites it is
// the next launch (pool_r4_carry_kernel).
template <int SA, int DPLA, int DPLI>
__global__ void __launch_bounds__(64 * (SA + 1)) pool_r4_kernel(PoolArgs a) {
  __shared__ float s_ss[SA];
  if (a.k_lo + (int64_t)blockIdx.x >= a.k_hi) return;  // a call without windows launches one empty workgroup
  r4_window<SA, DPLA, DPLI>(a, a.k_lo + blockIdx.x, s_ss);
}

__global__ void __launch_bounds__(256) pool_r4_carry_kernel(PoolArgs a) {
  carry_frontier_wide<4>(a, blockIdx.x, gridDim.x);
}

// Ratio 128, phase 1: workgroup (row, 64-dim slice, 64-token half) pools 64
// tokens x 64 dims (16 dim groups of 4 x 16 token groups of 4), merges the
// 16 groups through LDS and writes the (max, sum, weighted sum) partial of
// each dim: part[row][half][0..2][D].
__global__ void __launch_bounds__(256) pool_r128_partial_kernel(PoolArgs a) {
  __shared__ float s_m[16][64], s_s[16][64], s_a[16][64];
  const LaneDev& L = a.lane[0];
  const int S = L.D / 64;
  const int half = blockIdx.x & 1;
  const int slice = (blockIdx.x >> 1) % S;
  const int64_t row = (blockIdx.x >> 1) / S;
  if (row >= a.k_hi - a.k_lo) return;  // a call without windows launches one empty workgroup
  const int64_t k = a.k_lo + row;
  const int tid = threadIdx.x;
  const int dg = tid & 15, tg = tid >> 4;
  const int c = slice * 64 + dg * 4;
  float kv[4][4], sc[4][4];
#pragma unroll
  for (int e = 0; e < 4; ++e) fetch_token<128, 4>(a, L, 128 * k + 64 * half + tg + 16 * e, c, kv[e], sc[e]);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float m = sc[0][i];
#pragma unroll
    for (int e = 1; e < 4; ++e) m = fmaxf(m, sc[e][i]);
    float den = 0.f, num = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w = pool_exp(sc[e][i] - m);
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
          const float f = pool_exp(mg - M);
          den = fmaf(s_s[g][tid], f, den);
          num = fmaf(s_a[g][tid], f, num);
        }
      }
    }
    float* out = a.part + ((row * 2 + half) * 3) * L.D + slice * 64 + tid;
    out[0] = M;
    out[L.D] = den;
    out[2 * L.D] = num;
  }
}

// Ratio 128, phase 2: one wave per row merges the two halves' partials and
// finishes the row; workgroup 0 then carries the frontier.
template <int DPL>
__global__ void __launch_bounds__(256) pool_r128_finish_kernel(PoolArgs a) {
  const LaneDev& L = a.lane[0];
  const int row_groups = (int)((a.k_hi - a.k_lo + 3) / 4);
  if ((int)blockIdx.x >= row_groups) {
    // The partial-pool launch was the last reader of the incoming frontier.
    carry_frontier_wide<128>(a, blockIdx.x - row_groups, gridDim.x - row_groups);
    return;
  }
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * 4 + wave;
  if (row < a.k_hi - a.k_lo) {
    const int d0 = lane * DPL;
    float nw[DPL];
    load_vec<DPL>(nw, L.norm_w + d0);
    float M[DPL], den[DPL], num[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) { M[i] = -INFINITY; den[i] = 0.f; num[i] = 0.f; }
    float m[2][DPL], s[2][DPL], acc[2][DPL];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float* p = a.part + ((row * 2 + h) * 3) * L.D + d0;
      load_vec<DPL>(m[h], p);
      load_vec<DPL>(s[h], p + L.D);
      load_vec<DPL>(acc[h], p + 2 * L.D);
#pragma unroll
      for (int i = 0; i < DPL; ++i) M[i] = fmaxf(M[i], m[h][i]);
    }
    float o[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      if (M[i] != -INFINITY) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          if (m[h][i] == -INFINITY) continue;
          const float f = pool_exp(m[h][i] - M[i]);
          den[i] = fmaf(s[h][i], f, den[i]);
          num[i] = fmaf(acc[h][i], f, num[i]);
        }
      }
      o[i] = den[i] > 0.f ? num[i] / den[i] : 0.f;
    }
    const int64_t k = a.k_lo + row;
    float* pre = L.prequant ? L.prequant + row * L.D : nullptr;
    const RowConsts<DPL> rc = row_consts<DPL>(d0, L.D, a.n_rot, a.log2_base, k, 128);
    finish_row_wave<DPL>(o, nw, L, a.n_rot, a.rms_eps, rc, pre, L.rows + k * L.D, lane);
  }
}


// ---------------------------------------------------------------------------
// Fused ratio 4 (calls with n0 % 4 == 0): the projection epilogue has pooled
// every window j = k - k_lo with j % 64 != 0 into o[j][dim] (attention dims,
// then indexer dims) and left, for the windows j % 64 == 0, the previous and
// current halves' (max, sum, weighted sum) partials in part[j/64][0] and
// part[j/64][1] (window 0's previous half comes from the incoming frontier,
// read by the projection launch).
// ---------------------------------------------------------------------------
// mid() runs once the loads are issued and before their data is used.
template <int DPL, typename Mid>
__device__ __forceinline__ void fused_pool_dims(const PoolArgs& a, int64_t j, int dg, float (&o)[DPL], Mid&& mid) {
  if (j % 64 != 0) {
    load_vec<DPL>(o, a.o + j * a.d_tot + dg);
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
    return;
  }
  const int64_t tm = j / 64;
  float mc[DPL], sc[DPL], wc[DPL], mp[DPL], sp[DPL], wp[DPL];
  const float* pc = a.part + (tm * 2 + 1) * 3 * a.d_tot + dg;
  const float* pp = a.part + (tm * 2) * 3 * a.d_tot + dg;
  load_vec<DPL>(mc, pc);
  load_vec<DPL>(sc, pc + a.d_tot);
  load_vec<DPL>(wc, pc + 2 * a.d_tot);
  load_vec<DPL>(mp, pp);
  load_vec<DPL>(sp, pp + a.d_tot);
  load_vec<DPL>(wp, pp + 2 * a.d_tot);
  __builtin_amdgcn_sched_barrier(0);
  mid();
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    const float m = fmaxf(mc[i], mp[i]);
    float den = 0.f, num = 0.f;
    if (m != -INFINITY) {
      if (mc[i] != -INFINITY) {
        const float f = pool_exp(mc[i] - m);
        den = sc[i] * f;
        num = wc[i] * f;
      }
      if (mp[i] != -INFINITY) {
        const float f = pool_exp(mp[i] - m);
        den = fmaf(sp[i], f, den);
        num = fmaf(wp[i], f, num);
      }
    }
    o[i] = den > 0.f ? num / den : 0.f;
  }
}

template <int SA, int DPLA, int DPLI>
__device__ __forceinline__ void r4_fused_window(const PoolArgs& a, int64_t j, float* s_ss) {
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int64_t k = a.k_lo + j;
  if (wave < SA) {
    const LaneDev& L = a.lane[0];
    const int d0 = wave * (kWave * DPLA) + lane * DPLA;
    float nw[DPLA], o[DPLA];
    load_vec<DPLA>(nw, L.norm_w + d0);
    // The row constants need none of the loads: computed while they are in flight.
    RowConsts<DPLA> rc;
    fused_pool_dims<DPLA>(a, j, d0, o, [&] { rc = row_consts<DPLA>(d0, L.D, a.n_rot, a.log2_base, k, 4); });
    const float ss = wave_sum(row_sumsq<DPLA>(o));
    if (lane == 0) s_ss[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int s = 0; s < SA; ++s) tot += s_ss[s];
    float* pre = L.prequant ? L.prequant + j * L.D : nullptr;
    finish_row_part<DPLA>(o, nw, L, rms_inv(tot, L.D, a.rms_eps), d0, a.n_rot, rc, pre, L.rows + k * L.D, lane);
  } else {
    const LaneDev& L = a.lane[1];
    float nw[DPLI], o[DPLI];
    load_vec<DPLI>(nw, L.norm_w + lane * DPLI);
    RowConsts<DPLI> rc;
    fused_pool_dims<DPLI>(a, j, a.lane[0].D + lane * DPLI, o,
                          [&] { rc = row_consts<DPLI>(lane * DPLI, L.D, a.n_rot, a.log2_base, k, 4); });
    __syncthreads();
    float* pre = L.prequant ? L.prequant + j * L.D : nullptr;
    finish_row_wave<DPLI>(o, nw, L, a.n_rot, a.rms_eps, rc, pre, L.rows + k * L.D, lane);
  }
}

// Workgroups 0 .. n_emit-1 finish one window each; the kFusedCarryGroups
// after them write the outgoing frontier from the staged tokens (the
// projection launch was the last reader of the incoming one): with
// m = T - T % 4 (call-relative), rows 0..3 take tokens m-4 .. m-1 when m >= 4
// and rows 4.. take tokens m .. T-1.  32 groups give each thread one or two
// 16-byte copies (each a dependent load and store), so the carry is not the
// last workgroup to finish (4 groups: 5.0 us per launch, 32: 4.6 us).
constexpr int kFusedCarryGroups = 32;

template <int SA, int DPLA, int DPLI>
__global__ void __launch_bounds__(64 * (SA + 1)) pool_r4_fused_kernel(PoolArgs a) {
  __shared__ float s_ss[SA];
  const int64_t n_emit = a.k_hi - a.k_lo;
  if ((int64_t)blockIdx.x < n_emit) {
    r4_fused_window<SA, DPLA, DPLI>(a, blockIdx.x, s_ss);
    return;
  }
  const int64_t m = a.T - (a.T & 3);
  const int64_t first = m >= 4 ? m - 4 : 0;
  const int n_tok = (int)(a.T - first);
  // Flat work list: per lane, per kept token, kv then score, W/4 float4 each.
  const int64_t gid = (blockIdx.x - n_emit) * (int64_t)blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)kFusedCarryGroups * blockDim.x;
  int64_t base = 0;
  for (int l = 0; l < a.n_lanes; ++l) {
    const LaneDev& L = a.lane[l];
    const int w4 = L.W / 4;
    const int64_t count = (int64_t)n_tok * 2 * w4;
    for (int64_t i = gid - base; i < count; i += stride) {
      if (i < 0) continue;
      const int c = (int)(i % w4) * 4;
      const int kind = (int)((i / w4) & 1);
      const int64_t t = first + i / (2 * w4);
      const int row = t >= m ? 4 + (int)(t & 3) : (int)(t & 3);
      const float* src = a.stage + (t - a.carry_lo) * a.ld + (kind ? L.sc_col : L.kv_col) + c;
      float* dst = (kind ? L.fr_sc : L.fr_kv) + row * L.W + c;
      *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
    }
    base += count;
  }
}


// Fused ratio 128 (calls with n0 % 128 == 0): the projection epilogue has
// pooled window j into o[j][D].  One wave finishes one row; the
// kFusedCarryGroups workgroups after the rows write the outgoing frontier:
// rows 0 .. c-1 take the trailing partial window's tokens m .. T-1.
template <int DPL>
__global__ void __launch_bounds__(256) pool_r128_fused_kernel(PoolArgs a) {
  const LaneDev& L = a.lane[0];
  const int64_t n_emit = a.k_hi - a.k_lo;
  const int64_t row_groups = (n_emit + 3) / 4;
  if ((int64_t)blockIdx.x < row_groups) {
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    const int64_t j = (int64_t)blockIdx.x * 4 + wave;
    if (j < n_emit) {
      float nw[DPL], o[DPL];
      load_vec<DPL>(nw, L.norm_w + lane * DPL);
      load_vec<DPL>(o, a.o + j * L.D + lane * DPL);
      const int64_t k = a.k_lo + j;
      __builtin_amdgcn_sched_barrier(0);
      const RowConsts<DPL> rc = row_consts<DPL>(lane * DPL, L.D, a.n_rot, a.log2_base, k, 128);  // while the row loads
      __builtin_amdgcn_sched_barrier(0);
      float* pre = L.prequant ? L.prequant + j * L.D : nullptr;
      finish_row_wave<DPL>(o, nw, L, a.n_rot, a.rms_eps, rc, pre, L.rows + k * L.D, lane);
    }
    return;
  }
  const int64_t m = a.T - (a.T & 127);
  const int w4 = L.W / 4;
  const int64_t count = (a.T - m) * 2 * w4;
  const int64_t gid = (blockIdx.x - row_groups) * (int64_t)blockDim.x + threadIdx.x;
  for (int64_t i = gid; i < count; i += (int64_t)kFusedCarryGroups * blockDim.x) {
    const int c = (int)(i % w4) * 4;
    const int kind = (int)((i / w4) & 1);
    const int64_t t = m + i / (2 * w4);
    const float* src = a.stage + (t - a.carry_lo) * a.ld + (kind ? L.sc_col : L.kv_col) + c;
    float* dst = (kind ? L.fr_sc : L.fr_kv) + (t - m) * L.W + c;
    *reinterpret_cast<float4*>(dst) = *reinterpret_cast<const float4*>(src);
  }
}

__global__ void __launch_bounds__(256) frontier_fill_kernel(FillArgs f) {
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

template <int SA, int DPLA, int DPLI>
void launch_r4_one(const PoolArgs& a, unsigned grid, hipStream_t s, const Timing& tm) {
  const dim3 block(64 * (SA + 1));
  if (a.o)
    hipExtLaunchKernelGGL((pool_r4_fused_kernel<SA, DPLA, DPLI>), dim3(grid), block, 0, s, tm.start, tm.stop, 0, a);
  else
    hipExtLaunchKernelGGL((pool_r4_kernel<SA, DPLA, DPLI>), dim3(grid), block, 0, s, tm.start, tm.stop, 0, a);
}

template <int SA, int DPLA>
void launch_r4_a(const PoolArgs& a, int dpli, unsigned grid, hipStream_t s, const Timing& tm) {
  switch (dpli) {
    case 1: launch_r4_one<SA, DPLA, 1>(a, grid, s, tm); break;
    case 2: launch_r4_one<SA, DPLA, 2>(a, grid, s, tm); break;
    case 4: launch_r4_one<SA, DPLA, 4>(a, grid, s, tm); break;
    default: launch_r4_one<SA, DPLA, 8>(a, grid, s, tm); break;
  }
}

}  // namespace

int pool_launches(const PoolArgs& a) { return a.o ? 1 : 2; }

hipError_t launch_pool(const PoolArgs& a, int phase, hipStream_t stream, const Timing& tm) {
  const int64_t n_rows = a.k_hi - a.k_lo;
  if (a.ratio == 4 && !a.o && phase == 1) {
    hipExtLaunchKernelGGL(pool_r4_carry_kernel, dim3(carry_groups(a)), dim3(256), 0, stream, tm.start, tm.stop, 0, a);
  } else if (a.ratio == 4) {
    // Attention rows are split into waves of 256 dims at D = 512 (two waves,
    // four dims per lane: 5 % faster than four waves of 128 dims), 128 dims
    // at D = 128 / 256, 64 dims at D = 64.  Every launch is made, empty or
    // not, so that profiling brackets stay whole.
    const unsigned grid = a.o ? (unsigned)(n_rows + kFusedCarryGroups) : (unsigned)(n_rows > 0 ? n_rows : 1);
    const int da = a.lane[0].D, dpli = a.lane[1].D / 64;
    switch (da) {
      case 64: launch_r4_a<1, 1>(a, dpli, grid, stream, tm); break;
      case 128: launch_r4_a<1, 2>(a, dpli, grid, stream, tm); break;
      case 256: launch_r4_a<2, 2>(a, dpli, grid, stream, tm); break;
      default: launch_r4_a<2, 4>(a, dpli, grid, stream, tm); break;
    }
  } else if (a.o) {
    const unsigned grid = (unsigned)((n_rows + 3) / 4 + kFusedCarryGroups);
    switch (a.lane[0].D / 64) {
      case 1: hipExtLaunchKernelGGL((pool_r128_fused_kernel<1>), dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a); break;
      case 2: hipExtLaunchKernelGGL((pool_r128_fused_kernel<2>), dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a); break;
      case 4: hipExtLaunchKernelGGL((pool_r128_fused_kernel<4>), dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a); break;
      default: hipExtLaunchKernelGGL((pool_r128_fused_kernel<8>), dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a); break;
    }
  } else if (phase == 0) {
    const unsigned grid = (unsigned)(n_rows > 0 ? n_rows * (a.lane[0].D / 64) * 2 : 1);
    hipExtLaunchKernelGGL(pool_r128_partial_kernel, dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a);
  } else {
    const unsigned grid = (unsigned)((n_rows + 3) / 4 + carry_groups(a));
    switch (a.lane[0].D / 64) {
      case 1: hipExtLaunchKernelGGL((pool_r128_finish_kernel<1>), dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a); break;
      case 2: hipExtLaunchKernelGGL((pool_r128_finish_kernel<2>), dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a); break;
      case 4: hipExtLaunchKernelGGL((pool_r128_finish_kernel<4>), dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a); break;
      default: hipExtLaunchKernelGGL((pool_r128_finish_kernel<8>), dim3(grid), dim3(256), 0, stream, tm.start, tm.stop, 0, a); break;
    }
  }
  return hipGetLastError();
}

// Cache eviction for cold timings: reads (kWrite = false) or writes n16
// 16-byte words of a caller-owned buffer, displacing whatever the caches
// held.  Read lines stay clean; written lines are dirty and cost a write-back
// when the next kernel displaces them.  The read form stores only if the
// XOR of everything it read equals the word's index, so the loads stay live.
template <bool kWrite>
__global__ void __launch_bounds__(256) evict_kernel(uint4* p, int64_t n16) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t i0 = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (int64_t i = i0; i < n16; i += stride) {
    if constexpr (kWrite) {
      p[i] = make_uint4((uint32_t)i, 0u, 0u, 0u);
    } else {
      const uint4 v = p[i];
      acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if (!kWrite && i0 < n16 && acc == (uint32_t)i0 + 0x9e3779b9u) p[i0].x = acc;
}

hipError_t launch_evict(void* p, size_t bytes, bool write, hipStream_t stream) {
  if (write)
    hipLaunchKernelGGL(evict_kernel<true>, dim3(2048), dim3(256), 0, stream, static_cast<uint4*>(p),
                       (int64_t)(bytes / 16));
  else
    hipLaunchKernelGGL(evict_kernel<false>, dim3(2048), dim3(256), 0, stream, static_cast<uint4*>(p),
                       (int64_t)(bytes / 16));
  return hipGetLastError();
}

hipError_t launch_fill(const FillArgs& f, hipStream_t stream, const Timing& tm) {
  hipExtLaunchKernelGGL(frontier_fill_kernel, dim3(64), dim3(256), 0, stream, tm.start, tm.stop, 0, f);
  return hipGetLastError();
}

}  // namespace ds4c
