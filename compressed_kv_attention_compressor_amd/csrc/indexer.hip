// Indexer scoring and top-k over a layer's compressed indexer rows (Part 3
// §6: 64 indexer heads of 128 dims score the compressed rows and the top 512
// reach the attention; Part 3 §9: the query passes the same Hadamard + FP4
// round trip as the rows).  One query token per call.
//
// score(j) = sum_h w_h * max(0, <qhat_h, k_j>), qhat_h the QAT round trip of
// head h's query (rows and query both stay in the rotated basis).  The top-k
// order is descending score, equal scores to the lower row index.
//
// Launches:
//  * indexer_score_kernel: at most one workgroup per CU, each taking 64-row
//    blocks in turn.  The workgroup rotates and quantises the query into LDS
//    (each wave a quarter of the heads) while its first rows load; the dot
//    products run on bf16 MFMA tiles of 32 rows x 32 heads, one per wave, the
//    rows split into two bf16 parts, and the heads' weighted sum meets in a
//    fixed order.
//  * indexer_select_kernel: the k largest (score, lower row first) by a radix
//    select over 64-bit keys in one workgroup, the survivors then sorted
//    descending.  Up to kIndexerChunk rows it is one launch; longer calls run
//    one workgroup per chunk first and a final pass over their survivors.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace ds4c {

namespace {

constexpr int kScoreRows = 64;
constexpr int kScoreThreads = 256;  // also one thread per first-digit bin
constexpr int kScoreGrid = 256;     // score workgroups at most: one per CU
constexpr int kHistGroups = 16;     // select threads summing one word of a chunk's block counts
constexpr int kHistPerThread = kIndexerChunk / kScoreRows / kHistGroups;
constexpr int kSortThreads = 1024;
constexpr int kSelPerThread = kIndexerChunk / kSortThreads;  // keys per thread in a select pass

// Order-preserving map of float bits to unsigned: larger float, larger key.
__device__ __forceinline__ uint32_t ord_bits(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float unord_bits(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7fffffffu) : ~o);
}

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Eight floats as bf16 rounded to nearest even (hi) and their remainders,
// which are exact in float, rounded to bf16 again (lo).  Rounding to bf16's
// 8 significant bits errs by at most 2^-8 of the value, so |x - hi| <=
// 2^-8 |x| and x = hi + lo to within 2^-16 |x|; exactly when x has at most 8
// significant bits (as every value of an FP4 row with its power-of-two
// scale has).
__device__ __forceinline__ void split_bf16(const float4& a, const float4& b, bf16x8& hi, bf16x8& lo) {
  const f32x8 x = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  hi = __builtin_convertvector(x, bf16x8);
  lo = __builtin_convertvector(x - __builtin_convertvector(hi, f32x8), bf16x8);
}

// The heads' dot products with the rows are a [heads x Dh] x [Dh x rows]
// product: wave w takes rows 32 (w & 1) .. +31 of a 64-row block against
// heads 32 (w >> 1) .. +31 as one 32 x 32 tile of bf16 MFMAs with float
// accumulation (v_mfma_f32_32x32x16_bf16; its result holds, in lane l, row
// l % 32 against heads 8 (v / 4) + 4 (l / 32) + v % 4 of the tile, v =
// 0..15).  The query after its FP4 round trip is exact in bf16; each row
// value is split into two bf16 parts (split_bf16), multiplied separately and
// summed in float, so a score differs from a float dot product only by the
// split's 2^-16 and the order of the float additions (FP4 rows, which the
// compressor writes, split exactly).  The sum runs over the dims in an order
// of the kernel's choosing, the same on both operands: lane half h = l / 32
// takes dims Dh/2 * h .. +Dh/2 - 1, eight per MFMA, so each lane reads one
// contiguous half row from memory straight into its operand registers, and
// its query operands come from LDS eight dims per 16-byte read.  A
// workgroup rotates the query once and then takes the 64-row blocks
// blockIdx.x, blockIdx.x + gridDim.x, ... (the grid is at most one
// workgroup per CU), loading each block's rows while the previous block's
// MFMAs run.
template <int DH>
__global__ void __launch_bounds__(kScoreThreads) indexer_score_kernel(IndexerArgs a) {
  constexpr int kLd = DH + 8;   // padded bf16 LDS row: consecutive heads 16 bytes apart in the banks
  constexpr int kHalf = DH / 2; // dims per lane half
  constexpr int kV = kHalf / 4; // float4 per lane
  __shared__ __attribute__((aligned(16))) __bf16 s_q[64 * kLd];
  __shared__ float s_part[2][kScoreRows];
  __shared__ uint32_t s_hist[2][256];  // by block parity
  const int t = threadIdx.x, wave = t / kWave, lane = t % kWave;
  const int h = lane >> 5, r32 = lane & 31;
  const int rb = 32 * (wave & 1), hb = 32 * (wave >> 1);
  const int64_t n_blocks = (a.n + kScoreRows - 1) / kScoreRows;

  // This lane's half row of the block's row rb + r32 (rows past n re-read
  // row n-1; their scores are not written).
  auto load_rows = [&](float4 (&kv)[kV], int64_t blk) {
    const int64_t r = blk * kScoreRows + rb + r32;
    const int64_t row = r < a.n ? r : a.n - 1;
#pragma unroll
    for (int u = 0; u < kV; ++u) kv[u] = *reinterpret_cast<const float4*>(a.rows + row * DH + kHalf * h + 4 * u);
  };

  // Every load is issued before any is used, with no branch around a load
  // (a branch would make the compiler wait for each load before the next):
  // first the wave's query heads wave + 4m (m = 0..15; heads past H re-read
  // head H-1 and are zeroed), then the first block's rows and the weights of
  // this lane's 16 heads.  Loads complete in order, so the query's round trip
  // below waits only for the query.  For the round trip a head spans kLH
  // lanes of 8 dims each, so three of its butterfly stages stay inside a
  // lane.
  constexpr int kLH = DH / 8;            // lanes per head
  constexpr int kHPass = kWave / kLH;    // heads side by side in the wave
  constexpr int kSlots = 16 / kHPass;    // heads per lane
  const int hgrp = lane / kLH, dcol = 8 * (lane % kLH);
  float y[kSlots][8];
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int hq = wave + 4 * (kHPass * j + hgrp);
    load_vec<8>(y[j], a.q + (hq < a.H ? hq : a.H - 1) * DH + dcol);
  }
  float4 kv[kV];
  load_rows(kv, blockIdx.x);
  float w[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) {
    const int hd = hb + 8 * (v / 4) + 4 * h + v % 4;
    w[v] = a.head_w[hd < a.H ? hd : a.H - 1];
  }
  // Keeps the compiler from moving the row loads down to their first use,
  // past the query's round trip.
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int j = 0; j < kSlots; ++j)
    if (wave + 4 * (kHPass * j + hgrp) >= a.H)
#pragma unroll
      for (int i = 0; i < 8; ++i) y[j][i] = 0.f;
  // Rotation + FP4 round trip of the wave's heads into LDS (a zero head
  // stays zero), while the rows are still on their way.
  hadamard_fp4_rows<8, kSlots, kLH>(y, hadamard_scale(DH), lane);
#pragma unroll
  for (int j = 0; j < kSlots; ++j) {
    const int hq = wave + 4 * (kHPass * j + hgrp);
    const f32x8 yv = {y[j][0], y[j][1], y[j][2], y[j][3], y[j][4], y[j][5], y[j][6], y[j][7]};
    *reinterpret_cast<bf16x8*>(s_q + hq * kLd + dcol) = __builtin_convertvector(yv, bf16x8);  // exact
    if (a.q_hat && blockIdx.x == 0 && hq < a.H) store_vec<8>(a.q_hat + hq * DH + dcol, y[j]);
  }
#pragma unroll
  for (int v = 0; v < 16; ++v)
    if (hb + 8 * (v / 4) + 4 * h + v % 4 >= a.H) w[v] = 0.f;
  s_hist[0][t] = 0u;
  __syncthreads();

  const __bf16* qrow = s_q + (hb + r32) * kLd + kHalf * h;
  int par = 0;
  for (int64_t blk = blockIdx.x; blk < n_blocks; blk += gridDim.x, par ^= 1) {
    // The next block's rows load while this block's MFMAs run.
    const bool has_next = blk + gridDim.x < n_blocks;
    float4 kv_next[kV];
    if (has_next) load_rows(kv_next, blk + gridDim.x);
    // The rows' two bf16 parts accumulate apart (which also keeps
    // consecutive MFMAs independent) and are added once at the end.
    f32x16 acc0 = {}, acc1 = {};
#pragma unroll
    for (int st = 0; st < kV / 2; ++st) {
      const bf16x8 q8 = *reinterpret_cast<const bf16x8*>(qrow + 8 * st);
      bf16x8 khi, klo;
      split_bf16(kv[2 * st], kv[2 * st + 1], khi, klo);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q8, khi, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(q8, klo, acc1, 0, 0, 0);
    }
    // Weighted ReLU sum over the lane's 16 heads, then over the other lane
    // half (the tile's other 16 heads), then over the two head tiles in
    // LDS, each in a fixed order.
    float sc = 0.f;
#pragma unroll
    for (int v = 0; v < 16; ++v) sc = fmaf(w[v], fmaxf(acc0[v] + acc1[v], 0.f), sc);
    sc += lane_xor(sc, 32);
    if (h == 0) s_part[wave >> 1][rb + r32] = sc;
    __syncthreads();
    // The select's first radix digit is the top byte of a key, which is the
    // top byte of the score's order-preserving bits: each block's rows are
    // counted per byte value here, where the counting is spread over every
    // score workgroup, and the block's 256 counts (at most 64, one byte
    // each) are written.  The other parity's counts are cleared for the
    // next block (their last reads were before the barrier above).
    s_hist[par ^ 1][t] = 0u;
    const int64_t row0 = blk * kScoreRows;
    if (t < kScoreRows && row0 + t < a.n) {
      const float score = s_part[0][t] + s_part[1][t];
      a.scores[row0 + t] = score;
      atomicAdd(&s_hist[par][ord_bits(score) >> 24], 1u);
    }
    __syncthreads();
    if (t < 64)
      a.hist[blk * 64 + t] = s_hist[par][4 * t] | (s_hist[par][4 * t + 1] << 8) | (s_hist[par][4 * t + 2] << 16) |
                             (s_hist[par][4 * t + 3] << 24);
    if (has_next)
#pragma unroll
      for (int u = 0; u < kV; ++u) kv[u] = kv_next[u];
  }
}

// One workgroup selects the k largest of up to kIndexerChunk unique 64-bit
// keys (order-preserving score bits, then the complement of the row index):
// mode 0 builds them from scores[base ..] (base = kIndexerChunk per
// workgroup), mode 1 reads the surviving keys of every chunk from cand (0 =
// padding).  A radix select over 8-bit digits, most significant first,
// narrows the bucket holding the k-th key until the keys still needed are
// the whole bucket; the keys at or above that bucket's lowest value are then
// exactly the k largest.  final: they are sorted and written as (row,
// score), descending; else they go to cand in any order.
template <int MODE>
__global__ void __launch_bounds__(kSortThreads) indexer_select_kernel(IndexerArgs a, int final_pass) {
  constexpr int mode = MODE;
  __shared__ uint32_t hist[256];
  __shared__ uint32_t part[MODE == 0 ? kHistGroups : 1][256];
  __shared__ uint64_t sel[512];
  __shared__ unsigned long long s_prefix, s_mask, s_thresh;
  __shared__ int s_need, s_done, s_cnt;
  const int tid = threadIdx.x, lane = tid % kWave;
  const int64_t base = mode == 0 ? (int64_t)blockIdx.x * kIndexerChunk : 0;
  const int64_t left = a.n - base;
  const int count = mode == 0 ? (int)(left < kIndexerChunk ? left : kIndexerChunk) : a.n_chunks * a.k;
  // Loads without branches around them (a clamped address past the end,
  // zeroed afterwards), so all of a thread's loads are in flight at once.
  // Mode 0: the raw score bits (the keys are formed after every load is
  // issued); mode 1: the keys themselves.
  uint64_t key[kSelPerThread];
  uint32_t raw[MODE == 0 ? kSelPerThread : 1];
#pragma unroll
  for (int j = 0; j < kSelPerThread; ++j) {
    const int i = j * kSortThreads + tid;
    const int ic = i < count ? i : count - 1;
    if constexpr (MODE == 0)
      raw[j] = __float_as_uint(a.scores[base + ic]);
    else
      key[j] = a.cand[ic];
  }
  // Mode 0: the first digit's counts come from the chunk's 64-row blocks,
  // counted by the score kernel.  Thread (word q, group g) adds word q of
  // blocks g, g + 16, ... in two registers of 16-bit fields (even and odd
  // bins; at most 32 * 64 per field).
  uint32_t hw[kHistPerThread];
  const int hq = tid % 64, hg = tid / 64;
  const int n_hw = (count + kScoreRows - 1) / kScoreRows;
  if constexpr (MODE == 0) {
    const int64_t w0 = base / kScoreRows;
#pragma unroll
    for (int i = 0; i < kHistPerThread; ++i) {
      const int wi = hg + kHistGroups * i;
      hw[i] = a.hist[(w0 + (wi < n_hw ? wi : n_hw - 1)) * 64 + hq];
    }
  }
  // Every load above is in flight before the first is used.
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (MODE == 0) {
#pragma unroll
    for (int j = 0; j < kSelPerThread; ++j) {
      const uint32_t row = (uint32_t)(base + j * kSortThreads + tid);
      key[j] = ((uint64_t)ord_bits(__uint_as_float(raw[j])) << 32) | (uint64_t)(0xffffffffu - row);
    }
  }
#pragma unroll
  for (int j = 0; j < kSelPerThread; ++j)
    if (j * kSortThreads + tid >= count) key[j] = 0ull;
  if constexpr (MODE == 0) {
    uint32_t ev = 0u, od = 0u;
#pragma unroll
    for (int i = 0; i < kHistPerThread; ++i) {
      const uint32_t x = hg + kHistGroups * i < n_hw ? hw[i] : 0u;
      ev += x & 0x00ff00ffu;
      od += (x >> 8) & 0x00ff00ffu;
    }
    part[hg][4 * hq] = ev & 0xffffu;
    part[hg][4 * hq + 1] = od & 0xffffu;
    part[hg][4 * hq + 2] = ev >> 16;
    part[hg][4 * hq + 3] = od >> 16;
    __syncthreads();
    if (tid < 256) {
      uint32_t c = 0u;
#pragma unroll
      for (int g = 0; g < kHistGroups; ++g) c += part[g][tid];
      hist[tid] = c;
    }
  }
  if (tid == 0) {
    s_prefix = 0ull;
    s_mask = 0ull;
    s_need = a.k;
    s_done = 0;
  }
  for (int shift = 56; shift >= 0; shift -= 8) {
    // In mode 0 the first digit's counts are already in hist.
    const bool counted = MODE == 0 && shift == 56;
    if (!counted && tid < 256) hist[tid] = 0u;
    __syncthreads();
    const uint64_t prefix = s_prefix, mask = s_mask;
    // One LDS atomic per key still in the bucket.  (Counting each distinct
    // digit of a wave once, by ballots, was twice as slow on the first digit,
    // which most scores share: the ballot loop is serial.)
    if (!counted) {
#pragma unroll
      for (int j = 0; j < kSelPerThread; ++j)
        if (key[j] != 0ull && (key[j] & mask) == prefix) atomicAdd(&hist[(key[j] >> shift) & 0xffu], 1u);
    }
    __syncthreads();
    if (tid < kWave) {
      // Lane l holds bins 255-4l .. 252-4l; inclusive counts from the top.
      uint32_t c[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) c[b] = hist[255 - 4 * lane - b];
      const uint32_t csum = c[0] + c[1] + c[2] + c[3];
      // Inclusive scan over the lanes as a butterfly: a lane in the upper
      // half of each pair of blocks adds the lower block's total.
      uint32_t P = csum, tot = csum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t t = (uint32_t)lane_xor((int)tot, o);
        if (lane & o) P += t;
        tot += t;
      }
      const uint32_t E = P - csum;
      const uint32_t need = (uint32_t)s_need;
      if (lane == kWave - 1 && P < need) {
        // Fewer keys than k (only in the first round): take every key.
        s_thresh = 1ull;
        s_done = 1;
      }
      if (E < need && need <= P) {
        uint32_t cum = E;
        int b = 0;
        while (cum + c[b] < need) cum += c[b++];
        const int d = 255 - 4 * lane - b;
        const uint64_t np = prefix | ((uint64_t)d << shift);
        s_prefix = np;
        s_mask = mask | (0xffull << shift);
        s_need = (int)(need - cum);
        if (need - cum == c[b]) {
          s_thresh = np;
          s_done = 1;
        }
      }
    }
    __syncthreads();
    if (s_done) break;
  }
  const uint64_t thresh = s_thresh;
  if (tid == 0) s_cnt = 0;
  __syncthreads();
#pragma unroll
  for (int j = 0; j < kSelPerThread; ++j) {
    if (key[j] != 0ull && key[j] >= thresh) sel[atomicAdd(&s_cnt, 1)] = key[j];
  }
  __syncthreads();
  const int total = s_cnt;
  if (!final_pass) {
    for (int i = tid; i < a.k; i += kSortThreads) a.cand[(int64_t)blockIdx.x * a.k + i] = i < total ? sel[i] : 0ull;
    return;
  }
  // Descending order by a bitonic sort of the selected keys (padded with
  // zeros, below every key, to 512), one key per thread of the first eight
  // waves: 45 compare-exchange steps, the 39 between lanes of one wave by
  // lane exchanges, the 6 across waves through LDS.  Keys are unique, so the
  // order is.
  static_assert(kSortThreads >= 512, "one key per thread");
  const bool sorter = tid < 512;  // whole waves
  uint64_t v = sorter && tid < total ? sel[tid] : 0ull;
#pragma unroll
  for (int size = 2; size <= 512; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t w = 0ull;
      if (stride >= kWave) {
        __syncthreads();  // every read of the previous step is done
        if (sorter) sel[tid] = v;
        __syncthreads();
        if (sorter) w = sel[tid ^ stride];
      } else if (sorter) {
        const uint32_t lo = (uint32_t)lane_xor((int)(uint32_t)v, stride);
        const uint32_t hi = (uint32_t)lane_xor((int)(uint32_t)(v >> 32), stride);
        w = ((uint64_t)hi << 32) | lo;
      }
      // Blocks of `size` alternate direction so that the last merge sorts
      // descending; within a pair the lower index keeps the larger key in a
      // descending block.
      const bool desc = (tid & size) == 0;
      const bool lower = (tid & stride) == 0;
      const uint64_t hi_k = v > w ? v : w, lo_k = v > w ? w : v;
      v = lower == desc ? hi_k : lo_k;
    }
  }
  if (sorter && tid < total) {
    a.out_idx[tid] = (int32_t)(0xffffffffu - (uint32_t)(v & 0xffffffffu));
    a.out_score[tid] = unord_bits((uint32_t)(v >> 32));
  }
}

}  // namespace

// Scratch of the allocation-free indexer entry point: the row scores, the
// per-chunk candidate keys and the 64-row blocks' first-digit counts of
// the largest call the indexer accepts (1,048,576 rows at k = 512: 4 MiB of
// scores, 128 KiB of keys, 4 MiB of counts).  Each
// device holds its own copy until the process ends; every call on a device
// shares it.
static __device__ __align__(256) unsigned char scratch[kIndexerScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

}  // namespace

hipError_t indexer_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    // The array's host-side name is only a handle: its device address comes
    // from the runtime, once per device, with that device current.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t stream, const Timing& tm) {
  if (a.n <= 0) return hipSuccess;
  const int64_t n_blocks = (a.n + kScoreRows - 1) / kScoreRows;
  const unsigned g_score = (unsigned)(n_blocks < kScoreGrid ? n_blocks : kScoreGrid);
  if (a.Dh == 64)
    hipExtLaunchKernelGGL((indexer_score_kernel<64>), dim3(g_score), dim3(kScoreThreads), 0, stream, tm.start,
                          nullptr, 0, a);
  else
    hipExtLaunchKernelGGL((indexer_score_kernel<128>), dim3(g_score), dim3(kScoreThreads), 0, stream, tm.start,
                          nullptr, 0, a);
  if (a.n_chunks > 1) {
    hipExtLaunchKernelGGL(indexer_select_kernel<0>, dim3((unsigned)a.n_chunks), dim3(kSortThreads), 0, stream,
                          nullptr, nullptr, 0, a, 0);
    hipExtLaunchKernelGGL(indexer_select_kernel<1>, dim3(1), dim3(kSortThreads), 0, stream, nullptr, tm.stop, 0, a, 1);
  } else {
    hipExtLaunchKernelGGL(indexer_select_kernel<0>, dim3(1), dim3(kSortThreads), 0, stream, nullptr, tm.stop, 0, a, 1);
  }
  return hipGetLastError();
}

}  // namespace ds4c
