// Indexer scoring and top-k over a layer's compressed indexer rows (Part 3
// §6: 64 indexer heads of 128 dims score the compressed rows and the top 512
// reach the attention; Part 3 §9: the query passes the same Hadamard + FP4
// round trip as the rows).  One query token per call.
//
// score(j) = sum_h w_h * max(0, <qhat_h, k_j>), qhat_h the QAT round trip of
// head h's query (rows and query both stay in the rotated basis).  The top-k
// order is descending score, equal scores to the lower row index.
//
// Three launches:
//  * indexer_score_kernel: 64 rows per workgroup.  The workgroup rotates and
//    quantises the query into LDS (each wave a quarter of the heads), stages
//    its rows in LDS, and thread (row, head group) accumulates the dot
//    products of its row with heads g, g+4, ...; the four head groups of a
//    row meet by two shuffles in a fixed order.
//  * indexer_topk_chunk_kernel: one workgroup per 4096 scores sorts keys
//    (order-preserving score bits, then the complement of the row index) by
//    a bitonic network in LDS and keeps the k largest.
//  * indexer_topk_merge_kernel: one workgroup sorts every chunk's survivors
//    the same way and writes the k largest as (row, score).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"
#include "launch.h"

namespace ds4c {

namespace {

constexpr int kScoreRows = 64;
constexpr int kScoreThreads = 256;
constexpr int kSortThreads = 1024;

// Order-preserving map of float bits to unsigned: larger float, larger key.
__device__ __forceinline__ uint32_t ord_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unord_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

template <int DH>
__global__ void __launch_bounds__(kScoreThreads) indexer_score_kernel(IndexerArgs a) {
  constexpr int DPL = DH / 64;
  constexpr int kLd = DH + 4;  // padded LDS row: consecutive rows start on different banks
  __shared__ float s_q[64 * kLd];
  __shared__ float s_k[kScoreRows * kLd];
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int64_t row0 = (int64_t)blockIdx.x * kScoreRows;

  // Rows of this workgroup (zeros past n), 16 bytes per thread and step.
  constexpr int kVec = DH / 4;  // float4 per row
  for (int i = t; i < kScoreRows * kVec; i += kScoreThreads) {
    const int r = i / kVec, c = (i % kVec) * 4;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row0 + r < a.n) v = *reinterpret_cast<const float4*>(a.rows + (row0 + r) * DH + c);
    *reinterpret_cast<float4*>(s_k + r * kLd + c) = v;
  }
  // Query heads wave, wave+4, ...: rotation + FP4 round trip into LDS.
  for (int h = wave; h < a.H; h += kScoreThreads / kWave) {
    float y[DPL];
    load_vec<DPL>(y, a.q + h * DH + lane * DPL);
    hadamard_fp4<DPL>(y, DH, lane);
#pragma unroll
    for (int i = 0; i < DPL; ++i) s_q[h * kLd + lane * DPL + i] = y[i];
    if (a.q_hat && blockIdx.x == 0) store_vec<DPL>(a.q_hat + h * DH + lane * DPL, y);
  }
  __syncthreads();

  const int r = t / 4, g = t % 4;
  const int nh = a.H / 4;  // heads g, g+4, ... of this thread
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  for (int d = 0; d < DH; d += 4) {
    const float4 k = *reinterpret_cast<const float4*>(s_k + r * kLd + d);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i < nh) {
        const float4 q = *reinterpret_cast<const float4*>(s_q + (g + 4 * i) * kLd + d);
        float v = acc[i];
        v = fmaf(k.x, q.x, v);
        v = fmaf(k.y, q.y, v);
        v = fmaf(k.z, q.z, v);
        v = fmaf(k.w, q.w, v);
        acc[i] = v;
      }
    }
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (i < nh) s = fmaf(a.head_w[g + 4 * i], fmaxf(acc[i], 0.f), s);
  // Head groups 0..3 of a row sit in adjacent lanes: (s0 + s1) + (s2 + s3).
  s += __shfl_xor(s, 1, kWave);
  s += __shfl_xor(s, 2, kWave);
  if (g == 0 && row0 + r < a.n) a.scores[row0 + r] = s;
}

// Bitonic sort of M keys in LDS (M a power of two), descending: merge steps
// of block size 2, 4, .., M, compare-exchange at strides size/2 .. 1, blocks
// alternating direction until the last step sorts everything descending.
template <int THREADS>
__device__ __forceinline__ void bitonic_desc(uint64_t* keys, int M) {
  for (int size = 2; size <= M; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int p = threadIdx.x; p < M / 2; p += THREADS) {
        const int i = 2 * stride * (p / stride) + (p % stride);
        const int j = i + stride;
        const uint64_t ki = keys[i], kj = keys[j];
        const bool desc = (i & size) == 0;
        if (desc ? (ki < kj) : (ki > kj)) {
          keys[i] = kj;
          keys[j] = ki;
        }
      }
      __syncthreads();
    }
  }
}

__global__ void __launch_bounds__(kSortThreads) indexer_topk_chunk_kernel(IndexerArgs a) {
  __shared__ uint64_t keys[kIndexerChunk];
  const int64_t base = (int64_t)blockIdx.x * kIndexerChunk;
  for (int i = threadIdx.x; i < kIndexerChunk; i += kSortThreads) {
    const int64_t j = base + i;
    keys[i] = j < a.n ? ((uint64_t)ord_bits(a.scores[j]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)j) : 0ull;
  }
  __syncthreads();
  bitonic_desc<kSortThreads>(keys, kIndexerChunk);
  for (int i = threadIdx.x; i < a.k; i += kSortThreads) a.cand[(int64_t)blockIdx.x * a.k + i] = keys[i];
}

__global__ void __launch_bounds__(kSortThreads) indexer_topk_merge_kernel(IndexerArgs a, int m) {
  __shared__ uint64_t keys[kIndexerMaxCand];
  const int count = a.n_chunks * a.k;
  for (int i = threadIdx.x; i < m; i += kSortThreads) keys[i] = i < count ? a.cand[i] : 0ull;
  __syncthreads();
  bitonic_desc<kSortThreads>(keys, m);
  const int out = a.n < a.k ? (int)a.n : a.k;
  for (int i = threadIdx.x; i < out; i += kSortThreads) {
    const uint64_t key = keys[i];
    a.out_idx[i] = (int32_t)(0xffffffffu - (uint32_t)(key & 0xffffffffu));
    a.out_score[i] = unord_bits((uint32_t)(key >> 32));
  }
}

}  // namespace

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream, const Timing& tm) {
  if (a.n <= 0) return hipSuccess;
  const unsigned g_score = (unsigned)((a.n + kScoreRows - 1) / kScoreRows);
  const Timing t_first{tm.start, nullptr};
  if (a.Dh == 64)
    hipExtLaunchKernelGGL((indexer_score_kernel<64>), dim3(g_score), dim3(kScoreThreads), 0, stream, t_first.start,
                          nullptr, 0, a);
  else
    hipExtLaunchKernelGGL((indexer_score_kernel<128>), dim3(g_score), dim3(kScoreThreads), 0, stream, t_first.start,
                          nullptr, 0, a);
  hipExtLaunchKernelGGL(indexer_topk_chunk_kernel, dim3((unsigned)a.n_chunks), dim3(kSortThreads), 0, stream, nullptr,
                        nullptr, 0, a);
  int m = 1;
  while (m < a.n_chunks * a.k) m <<= 1;
  if (m < 2) m = 2;
  hipExtLaunchKernelGGL(indexer_topk_merge_kernel, dim3(1), dim3(kSortThreads), 0, stream, nullptr, tm.stop, 0, a, m);
  return hipGetLastError();
}

}  // namespace ds4c
