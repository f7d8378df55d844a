// Ratio-4 indexed mixed attention of one decode query (Part 3 §7): the
// query's heads attend, in one softmax, the raw sliding-window rows it can
// see and the compressed rows the indexer's top-k list selects (negative
// entries skipped, the walk ending at the first entry at or beyond the
// visible rows).  Each row is key and value for every head; logits are
// <q_h, row> / sqrt(D).
//
// Items: the n_raw visible raw rows (ascending position), then the k list
// entries.  Launches:
//  * mixed_attn_part_kernel, grid (ceil(items / 32), H / 4), 4 waves: wave
//    w takes 8 items x 4 heads.  Lane l holds dims [l*DPL, (l+1)*DPL) of the
//    8 rows and of the 4 heads' queries; the 32 (item, head) dot products
//    are reduced by a butterfly that halves the set at each of five shuffle
//    steps, so lanes 2i and 2i+1 end with the full logit of pair i.  The wave's softmax
//    partial (max, sum, weighted rows) per head meets the other waves' in
//    LDS, in a fixed order, and one partial per (split, head) goes to the
//    workspace.  The list entries and rows are requested before the wave
//    works out where the walk ends, so a call costs two memory round trips.
//  * mixed_attn_merge_kernel, one wave per (head, 128 dims): rescales the
//    splits' partials to a common max, adds them in split order and
//    normalises.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace ds4c {

namespace {

constexpr int kHeadsPerGroup = 4;
constexpr int kItemsPerWave = 8;
constexpr int kAttnWaves = 4;

// Butterfly transpose-reduction: 32 values per lane in; lanes 2i and 2i+1
// out with the sum over all 64 lanes of value i.  Step m (32 .. 2) keeps the
// half of the set whose index bit matches lane bit log2(m) and receives the
// partner's copy of it; the last step adds the two lanes of a pair.
__device__ __forceinline__ float transpose_reduce32(const float (&v)[32], int lane) {
  float a[16], b[8], c[4], d[2];
  {
    const bool hi = (lane & 32) != 0;
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const float mine = hi ? v[16 + t] : v[t], other = hi ? v[t] : v[16 + t];
      a[t] = mine + lane_xor(other, 32);
    }
  }
  {
    const bool hi = (lane & 16) != 0;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float mine = hi ? a[8 + t] : a[t], other = hi ? a[t] : a[8 + t];
      b[t] = mine + lane_xor(other, 16);
    }
  }
  {
    const bool hi = (lane & 8) != 0;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const float mine = hi ? b[4 + t] : b[t], other = hi ? b[t] : b[4 + t];
      c[t] = mine + lane_xor(other, 8);
    }
  }
  {
    const bool hi = (lane & 4) != 0;
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const float mine = hi ? c[2 + t] : c[t], other = hi ? c[t] : c[2 + t];
      d[t] = mine + lane_xor(other, 4);
    }
  }
  const bool hi = (lane & 2) != 0;
  const float mine = hi ? d[1] : d[0], other = hi ? d[0] : d[1];
  const float e = mine + lane_xor(other, 2);
  return e + lane_xor(e, 1);
}

template <int DPL>
__global__ void __launch_bounds__(kAttnWaves * kWave) mixed_attn_part_kernel(MixedAttnArgs a) {
  constexpr int D = DPL * kWave;
  __shared__ float s_p[kAttnWaves][kItemsPerWave * kHeadsPerGroup];
  __shared__ float s_m[kAttnWaves][kHeadsPerGroup], s_l[kAttnWaves][kHeadsPerGroup];
  __shared__ __attribute__((aligned(16))) float s_o[kAttnWaves][kHeadsPerGroup][D];
  const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
  const int h0 = blockIdx.y * kHeadsPerGroup;

  // Loads in two round trips: the heads' queries, this wave's list entries
  // (wave-uniform) and the scan for the end of the walk first, then the
  // rows.  A list item's row is read when 0 <= entry < visible
  // (<= n_comp, so in bounds); anything else reads the first query row
  // (always present) and is masked below.  Raw item i is ring row
  // ring_row0 + i, wrapped once (n_raw <= ring_cap).
  float q[kHeadsPerGroup][DPL];
#pragma unroll
  for (int h = 0; h < kHeadsPerGroup; ++h) load_vec<DPL>(q[h], a.q + (int64_t)(h0 + h) * D + lane * DPL);
  const int it0 = (blockIdx.x * kAttnWaves + wave) * kItemsPerWave;
  int ent[kItemsPerWave], e0[8];
  if (a.k > 0) {
    // Clamped addresses: every load is issued, none is branched around.
#pragma unroll
    for (int j = 0; j < kItemsPerWave; ++j)
      ent[j] = __builtin_amdgcn_readfirstlane(a.topk[min(max(it0 + j - a.n_raw, 0), a.k - 1)]);
#pragma unroll
    for (int r = 0; r < 8; ++r) e0[r] = a.topk[min(r * kWave + lane, a.k - 1)];
  } else {
#pragma unroll
    for (int j = 0; j < kItemsPerWave; ++j) ent[j] = -1;
#pragma unroll
    for (int r = 0; r < 8; ++r) e0[r] = -1;
  }
  float x[kItemsPerWave][DPL];
#pragma unroll
  for (int j = 0; j < kItemsPerWave; ++j) {
    const int item = it0 + j, t = item - a.n_raw;
    if (t < 0 || t >= a.k) ent[j] = -1;
    const int r = a.ring_row0 + item;
    const float* raw = a.ring + (int64_t)(r < a.ring_cap ? r : r - a.ring_cap) * D;
    const float* cmp = a.comp + (int64_t)ent[j] * D;
    const float* rp = item < a.n_raw ? raw : (ent[j] >= 0 && ent[j] < a.visible ? cmp : a.q);
    load_vec<DPL>(x[j], rp + lane * DPL);
  }
  // The walk ends at the first list entry at or beyond the visible rows:
  // every wave finds it on its own (the first 512 entries from the loads
  // above, any further ones eight per lane per pass), then a wave minimum.
  int cut = a.k;
#pragma unroll
  for (int r = 0; r < 8; ++r) {
    const int i = r * kWave + lane;
    if (i < a.k && e0[r] >= a.visible) cut = min(cut, i);
  }
  for (int base = 8 * kWave; base < a.k; base += 8 * kWave) {
    int e[8];
#pragma unroll
    for (int r = 0; r < 8; ++r) e[r] = a.topk[min(base + r * kWave + lane, a.k - 1)];
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      const int i = base + r * kWave + lane;
      if (i < a.k && e[r] >= a.visible) cut = min(cut, i);
    }
  }
  cut = min(cut, lane_xor(cut, 32));
  cut = min(cut, lane_xor(cut, 16));
  cut = min(cut, lane_xor(cut, 8));
  cut = min(cut, lane_xor(cut, 4));
  cut = min(cut, lane_xor(cut, 2));
  cut = min(cut, lane_xor(cut, 1));
  unsigned valid = 0;
#pragma unroll
  for (int j = 0; j < kItemsPerWave; ++j) {
    const int item = it0 + j, t = item - a.n_raw;
    if (item < a.n_raw || (t < cut && ent[j] >= 0)) valid |= 1u << j;
  }
  float v[kItemsPerWave * kHeadsPerGroup];
  {
#pragma unroll
    for (int j = 0; j < kItemsPerWave; ++j)
#pragma unroll
      for (int h = 0; h < kHeadsPerGroup; ++h) {
        float s = 0.f;
#pragma unroll
        for (int d = 0; d < DPL; ++d) s = fmaf(q[h][d], x[j][d], s);
        v[j * kHeadsPerGroup + h] = s;
      }
  }
  // Lanes 2i, 2i+1: logit of pair i = item * 4 + head.
  const int pair = lane >> 1;
  const float logit = transpose_reduce32(v, lane);
  const float s = (valid >> (pair / kHeadsPerGroup)) & 1u ? logit * a.scale : -INFINITY;
  // Per head over the wave's 8 items (lanes that differ in bits 3-5).
  float m = s;
  m = fmaxf(m, lane_xor(m, 8));
  m = fmaxf(m, lane_xor(m, 16));
  m = fmaxf(m, lane_xor(m, 32));
  const float p = m == -INFINITY ? 0.f : pool_exp(s - m);
  float l = p;
  l += lane_xor(l, 8);
  l += lane_xor(l, 16);
  l += lane_xor(l, 32);
  if ((lane & 1) == 0) s_p[wave][pair] = p;
  if ((lane & 1) == 0 && pair < kHeadsPerGroup) {
    s_m[wave][pair] = m;
    s_l[wave][pair] = l;
  }
  __syncthreads();

  // Weighted rows of this wave, rescaled to the workgroup's max per head.
  float o[kHeadsPerGroup][DPL];
#pragma unroll
  for (int h = 0; h < kHeadsPerGroup; ++h) {
    float mx = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    const float f = mx == -INFINITY ? 0.f : pool_exp(s_m[wave][h] - mx);
#pragma unroll
    for (int d = 0; d < DPL; ++d) o[h][d] = 0.f;
#pragma unroll
    for (int j = 0; j < kItemsPerWave; ++j) {
      const float pj = s_p[wave][j * kHeadsPerGroup + h] * f;
#pragma unroll
      for (int d = 0; d < DPL; ++d) o[h][d] = fmaf(pj, x[j][d], o[h][d]);
    }
    store_vec<DPL>(&s_o[wave][h][lane * DPL], o[h]);
  }
  __syncthreads();

  // The workgroup's partial: waves added in order.
  const int64_t split = blockIdx.x;
  for (int e = threadIdx.x; e < kHeadsPerGroup * D; e += blockDim.x) {
    const int h = e / D, dd = e % D;
    float acc = s_o[0][h][dd];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) acc += s_o[w][h][dd];
    a.part_o[(split * a.H + h0 + h) * D + dd] = acc;
  }
  if (threadIdx.x < kHeadsPerGroup) {
    const int h = threadIdx.x;
    float mx = s_m[0][h];
#pragma unroll
    for (int w = 1; w < kAttnWaves; ++w) mx = fmaxf(mx, s_m[w][h]);
    float sum = 0.f;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) sum += mx == -INFINITY ? 0.f : s_l[w][h] * pool_exp(s_m[w][h] - mx);
    a.part_m[split * a.H + h0 + h] = mx;
    a.part_l[split * a.H + h0 + h] = sum;
  }
}

// Merge, one wave per (head, 64*DPL-dim chunk of the row), 32 splits per
// pass: lane i < 32 loads split i's (max, sum) while every lane loads its
// dims of the 32 splits' weighted rows, all issued before any is used (one
// memory round trip per pass).  Passes merge online: the running max, sum
// and weighted row are rescaled when a pass raises the max.  Splits are
// added in order, so the result does not depend on timing.
template <int DPL>
__global__ void __launch_bounds__(kWave) mixed_attn_merge_kernel(MixedAttnArgs a) {
  constexpr int kPass = 32;
  const int h = blockIdx.x, lane = threadIdx.x;
  const int64_t d0 = (int64_t)blockIdx.y * kWave * DPL + lane * DPL;
  float mx = -INFINITY, sum = 0.f, o[DPL];
#pragma unroll
  for (int d = 0; d < DPL; ++d) o[d] = 0.f;
  for (int s0 = 0; s0 < a.n_split; s0 += kPass) {
    const int s = min(s0 + (lane % kPass), a.n_split - 1);
    const bool mine = lane < kPass && s0 + lane < a.n_split;
    const float ms = a.part_m[(int64_t)s * a.H + h], ls = a.part_l[(int64_t)s * a.H + h];
    float t[kPass][DPL];
#pragma unroll
    for (int i = 0; i < kPass; ++i) {
      const int si = min(s0 + i, a.n_split - 1);
      load_vec<DPL>(t[i], a.part_o + ((int64_t)si * a.H + h) * a.D + d0);
    }
    float mp = mine ? ms : -INFINITY;
#pragma unroll
    for (int k = 32; k > 0; k >>= 1) mp = fmaxf(mp, lane_xor(mp, k));
    const float mn = fmaxf(mx, mp);
    if (mn == -INFINITY) continue;  // nothing attended so far (uniform)
    const float r = mx == -INFINITY ? 0.f : pool_exp(mx - mn);
    const float f = mine && ms != -INFINITY ? pool_exp(ms - mn) : 0.f;
    sum = sum * r + wave_sum(mine ? ls * f : 0.f);
#pragma unroll
    for (int d = 0; d < DPL; ++d) o[d] *= r;
#pragma unroll
    for (int i = 0; i < kPass; ++i) {
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), i));  // 0 for splits past the end
#pragma unroll
      for (int d = 0; d < DPL; ++d) o[d] = fmaf(t[i][d], w, o[d]);
    }
    mx = mn;
  }
  const float inv = sum > 0.f ? 1.f / sum : 0.f;
#pragma unroll
  for (int d = 0; d < DPL; ++d) o[d] *= inv;
  store_vec<DPL>(a.out + (int64_t)h * a.D + d0, o);
}

template <int DPL>
void launch_attn(const MixedAttnArgs& a, hipStream_t stream, const Timing& tm) {
  const dim3 g1(a.n_split, a.H / kHeadsPerGroup);
  hipExtLaunchKernelGGL(mixed_attn_part_kernel<DPL>, g1, dim3(kAttnWaves * kWave), 0, stream, tm.start, nullptr, 0,
                        a);
  constexpr int kMergeDpl = DPL < 2 ? DPL : 2;
  hipExtLaunchKernelGGL(mixed_attn_merge_kernel<kMergeDpl>, dim3(a.H, DPL / kMergeDpl), dim3(kWave), 0, stream,
                        nullptr, tm.stop, 0, a);
}

}  // namespace

int mixed_attn_splits(int n_items) {
  const int per = kAttnWaves * kItemsPerWave;
  return n_items > 0 ? (n_items + per - 1) / per : 1;
}

hipError_t launch_mixed_attention(const MixedAttnArgs& a, hipStream_t stream, const Timing& tm) {
  switch (a.D) {
    case 64: launch_attn<1>(a, stream, tm); break;
    case 128: launch_attn<2>(a, stream, tm); break;
    case 256: launch_attn<4>(a, stream, tm); break;
    default: launch_attn<8>(a, stream, tm); break;
  }
  return hipGetLastError();
}

}  // namespace ds4c
