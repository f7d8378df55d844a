// One decode token through a compressed layer (Part 3 §4,
// compressor_decode_one; Part 3 §5, the ratio-4 frontier).
//
// Every token: a GEMV launch in which each workgroup computes two projected
// columns (dot products of weight rows with x) and stores them straight into
// frontier row (coff-1)*ratio + pos%ratio, adding APE[pos%ratio] to scores.
// Only when (pos+1) % ratio == 0 the frontier is pooled into row pos/ratio
// of each lane (norm, tail RoPE, codec): on ratio-4 layers one workgroup
// pools, shifts rows 4..7 to 0..3 and finishes the rows; on ratio-128 layers
// a wide launch pools the 128 rows and a one-wave launch finishes the row.
// Each of these reads all of its entries at once, so a boundary costs about
// one memory round trip per launch.
// The launch boundary orders the pool after every column store.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <climits>
#include <cstddef>

#include "device_common.h"
#include "launch.h"

namespace ds4c {

namespace {

// Four waves per workgroup, two projected columns per workgroup: wave w
// takes the w-th quarter of K for both columns, and the four partial sums
// meet in LDS in a fixed order.  The grid (N/2 workgroups) spreads evenly
// over the CUs; against one wave per pair of columns over all of K this cut
// a 30-layer token (15 ratio-4 + 15 ratio-128 GEMVs, weights streamed from
// HBM) from 154 to 144 us on one MI355X.
constexpr int kDecWaves = 4;
constexpr int kDecThreads = 64 * kDecWaves;
constexpr int kColsPerBlock = 2;

__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

// acc += dot(w, x) over one 16-byte step.
__device__ __forceinline__ float dot16(uint4 w, uint4 x, float acc, uint16_t) {
  acc = fmaf(bf16_lo(w.x), bf16_lo(x.x), acc); acc = fmaf(bf16_hi(w.x), bf16_hi(x.x), acc);
  acc = fmaf(bf16_lo(w.y), bf16_lo(x.y), acc); acc = fmaf(bf16_hi(w.y), bf16_hi(x.y), acc);
  acc = fmaf(bf16_lo(w.z), bf16_lo(x.z), acc); acc = fmaf(bf16_hi(w.z), bf16_hi(x.z), acc);
  acc = fmaf(bf16_lo(w.w), bf16_lo(x.w), acc); acc = fmaf(bf16_hi(w.w), bf16_hi(x.w), acc);
  return acc;
}
__device__ __forceinline__ float dot16(uint4 w, uint4 x, float acc, float) {
  acc = fmaf(__uint_as_float(w.x), __uint_as_float(x.x), acc);
  acc = fmaf(__uint_as_float(w.y), __uint_as_float(x.y), acc);
  acc = fmaf(__uint_as_float(w.z), __uint_as_float(x.z), acc);
  acc = fmaf(__uint_as_float(w.w), __uint_as_float(x.w), acc);
  return acc;
}

// Pointers here are global memory; the casts keep the loads and stores in
// their global form when a pointer's origin is hidden from the compiler
// (flat accesses would also count against the LDS wait counter).
template <typename T>
__device__ __forceinline__ const __attribute__((address_space(1))) T* gptr(const void* p) {
  return (const __attribute__((address_space(1))) T*)p;
}

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// 16 bytes of a weight row, loaded with the nontemporal hint: each weight is
// read once per token, so its lines should not displace cached data (x, the
// frontier rows).  Against plain loads this cut a 30-layer token of GEMVs
// (in a HIP graph) from 141.6 to 133.9 us on one MI355X.
template <typename Tin>
__device__ __forceinline__ uint4 load_stream(const Tin* p) {
  const v4u t = __builtin_nontemporal_load(gptr<v4u>(p));
  return uint4{t.x, t.y, t.z, t.w};
}

template <typename Tin>
__device__ __forceinline__ uint4 load_global(const Tin* p) {
  const v4u t = *gptr<v4u>(p);
  return uint4{t.x, t.y, t.z, t.w};
}

// Two dot products over k in [k0, k0 + kr) of weight rows w0, w1 with x,
// one wave.  Lane l takes 16-byte step l of every 64-step span; U spans are
// loaded (x straight from global memory, where it stays cache-resident for
// the whole grid) before any of them is used.  Steps past the range load a
// clamped in-range address and are zeroed, so the body has no branches.
// mid() runs before any load is used: in the single-pass form after all of
// the loads are issued, in the looped form before the loop.
template <typename Tin, int U, typename Mid>
__device__ __forceinline__ void wave_dot2(const Tin* __restrict__ w0, const Tin* __restrict__ w1,
                                          const Tin* __restrict__ x, int k0, int kr, int lane, float* d0,
                                          float* d1, Mid&& mid) {
  constexpr int kVec = 16 / (int)sizeof(Tin), kSpan = kWave * kVec;
  const int kend = k0 + kr;
  float a0 = 0.f, a1 = 0.f;
  if (kr == kSpan * U) {  // the usual shape (hidden 4096 bf16): one pass, nothing to mask
    uint4 xv[U], u[U], v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int k = k0 + i * kSpan + lane * kVec;
      xv[i] = load_global(x + k);
      u[i] = load_stream(w0 + k);
      v[i] = load_stream(w1 + k);
    }
    __builtin_amdgcn_sched_barrier(0);
    mid();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < U; ++i) {
      a0 = dot16(u[i], xv[i], a0, Tin{});
      a1 = dot16(v[i], xv[i], a1, Tin{});
    }
    *d0 = wave_sum(a0);
    *d1 = wave_sum(a1);
    return;
  }
  mid();
  for (int kb = k0; kb < kend; kb += kSpan * U) {
    uint4 xv[U], u[U], v[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const int k = min(kb + i * kSpan + lane * kVec, kend - kVec);
      xv[i] = load_global(x + k);
      u[i] = load_stream(w0 + k);
      v[i] = load_stream(w1 + k);
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
      const bool in = kb + i * kSpan + lane * kVec < kend;
      const uint4 z = {0u, 0u, 0u, 0u};
      const uint4 xi = in ? xv[i] : z;
      a0 = dot16(in ? u[i] : z, xi, a0, Tin{});
      a1 = dot16(in ? v[i] : z, xi, a1, Tin{});
    }
  }
  *d0 = wave_sum(a0);
  *d1 = wave_sum(a1);
}

// The decode GEMV's argument segment, laid out as its parameter list (the
// kernel reads the store targets from it by offset).
struct GemvKernargs {
  const void* x;
  const void* w[4];
  const float* ape_a;
  unsigned kc;
  int ape_i_off;
  GemvStore st;
};

// Projection of one token into its frontier row.  Workgroup b covers
// columns [2b, 2b+2); both lie in one column block (blocks have even sizes).
// Every argument before `st` (14 dwords) arrives preloaded in scalar
// registers: the workgroup picks its block with scalar selects and issues
// its weight, x and APE loads at once, without waiting on memory for an
// argument; the frontier row it stores to is read from `st` meanwhile.
// kc = K/64 | c1/64 << 10 | c2/64 << 17 | c3/64 << 24: block s starts at
// output column c_s (c_0 = 0; unused blocks start at N).  ape_a: the
// attention lane's APE row for this token (score block 1); the indexer
// lane's (score block 3) is ape_a + ape_i_off, or st.ape_i in the FAR form
// (used when the two rows are not within 2^31 floats of each other).
template <typename Tin, int U, bool FAR>
__global__ void __launch_bounds__(kDecThreads)
    decode_gemv_kernel(const void* x_, const void* w0_, const void* w1_, const void* w2_, const void* w3_,
                       const float* ape_a, unsigned kc, int ape_i_off, GemvStore st) {
  __shared__ float s_part[kDecWaves][kColsPerBlock];
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave), lane = tid % kWave;
  const int K = (int)(kc & 1023u) * 64, c1 = (int)((kc >> 10) & 127u) * 64, c2 = (int)((kc >> 17) & 127u) * 64,
            c3 = (int)(kc >> 24) * 64;
  const int c0 = blockIdx.x * kColsPerBlock;  // the grid covers N exactly
  const int sg = c0 >= c3 ? 3 : c0 >= c2 ? 2 : c0 >= c1 ? 1 : 0;
  const void* ws = sg == 3 ? w3_ : sg == 2 ? w2_ : sg == 1 ? w1_ : w0_;
  const int j = c0 - (sg == 3 ? c3 : sg == 2 ? c2 : sg == 1 ? c1 : 0);
  const float* as = sg == 1 ? ape_a : sg == 3 ? (FAR ? st.ape_i : ape_a + ape_i_off) : nullptr;
  const Tin* w0 = reinterpret_cast<const Tin*>(ws) + (int64_t)j * K;
  const Tin* x = reinterpret_cast<const Tin*>(x_);
  const int kr = K / kDecWaves;  // K is a multiple of 64, so kr is a whole number of 16-byte steps
  // The APE pair is read with a vector load (a zero offset the compiler
  // cannot see through), issued with the weight loads.
  typedef float f2 __attribute__((ext_vector_type(2)));
  int zero;
  asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
  const f2 add = (as && wave == 0) ? *gptr<f2>(as + j + zero) : f2{0.f, 0.f};
  // The store target is read from the argument segment after the weight
  // loads are issued and waited for there, while they are in flight: the
  // scalar load and its wait sit in one statement, so the compiler can
  // neither hoist the load nor place its wait ahead of the weight loads.
  float* ds = nullptr;
  auto mid = [&]() {
    const __attribute__((address_space(4))) char* p =
        (const __attribute__((address_space(4))) char*)__builtin_amdgcn_kernarg_segment_ptr() +
        offsetof(GemvKernargs, st) + offsetof(GemvStore, dst) + sizeof(float*) * sg;
    asm volatile("s_load_dwordx2 %0, %1, 0x0\n\ts_waitcnt lgkmcnt(0)" : "=s"(ds) : "s"(p) : "memory");
  };
  float v0, v1;
  wave_dot2<Tin, U>(w0, w0 + K, x, wave * kr, kr, lane, &v0, &v1, mid);
  if (lane == 0) {
    s_part[wave][0] = v0;
    s_part[wave][1] = v1;
  }
  __syncthreads();
  if (tid < kColsPerBlock) {
    float v = s_part[0][tid];
#pragma unroll
    for (int q = 1; q < kDecWaves; ++q) v += s_part[q][tid];
    *(__attribute__((address_space(1))) float*)(ds + j + tid) = v + (tid == 0 ? add.x : add.y);
  }
}

struct GemvLaunch {
  const void* x;
  const void* w[4];
  unsigned kc;
  const float* ape_a;
  int ape_i_off;
  bool far;  // the indexer APE row is read from st (not within 2^31 floats of the attention row)
  GemvStore st;
};

template <typename Tin>
void launch_gemv(const GemvLaunch& g, int K, unsigned grid, hipStream_t s, hipEvent_t start, hipEvent_t stop) {
  // Spans of 64 16-byte steps in a wave's quarter of K, all loaded at once
  // (up to 8; longer quarters loop).
  constexpr int kSpan = kWave * (16 / (int)sizeof(Tin));
  const int spans = (K / kDecWaves + kSpan - 1) / kSpan;
  const dim3 gr(grid), bl(kDecThreads);
#define DS4C_GEMV(U)                                                                                        \
  (g.far ? hipExtLaunchKernelGGL((decode_gemv_kernel<Tin, U, true>), gr, bl, 0, s, start, stop, 0, g.x, g.w[0],  \
                                 g.w[1], g.w[2], g.w[3], g.ape_a, g.kc, g.ape_i_off, g.st)                   \
         : hipExtLaunchKernelGGL((decode_gemv_kernel<Tin, U, false>), gr, bl, 0, s, start, stop, 0, g.x, g.w[0], \
                                 g.w[1], g.w[2], g.w[3], g.ape_a, g.kc, g.ape_i_off, g.st))
  if (spans <= 1) DS4C_GEMV(1);
  else if (spans <= 2) DS4C_GEMV(2);
  else if (spans <= 4) DS4C_GEMV(4);
  else DS4C_GEMV(8);
#undef DS4C_GEMV
}

// One thread's share of a ratio-4 boundary for dims [d0, d0+DPL) of lane L:
// load the window's 8 entries (rows 0..3 on columns [0, D), rows 4..7 on
// columns [D, 2D)) and rows 4..7 on columns [0, D), pool the entries into
// o, and apply the half shift to the same columns (rows 0..3 <- rows 4..7 on
// both halves).  The thread writes only addresses it has read itself, so
// the shift needs no synchronisation with other threads.
template <int DPL, typename Mid>
__device__ __forceinline__ void r4_pool_and_shift(const LaneDev& L, int d0, float (&o)[DPL], Mid&& mid) {
  float kv[8][DPL], sc[8][DPL], kvs[4][DPL], scs[4][DPL];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = (e < 4 ? 0 : L.D) + d0;
    load_vec<DPL>(kv[e], L.fr_kv + e * L.W + c);
    load_vec<DPL>(sc[e], L.fr_sc + e * L.W + c);
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    load_vec<DPL>(kvs[e], L.fr_kv + (e + 4) * L.W + d0);
    load_vec<DPL>(scs[e], L.fr_sc + (e + 4) * L.W + d0);
  }
  // Work that needs none of the loads runs while they are in flight.
  __builtin_amdgcn_sched_barrier(0);
  mid();
  __builtin_amdgcn_sched_barrier(0);
  pool_entries<8, DPL>(kv, sc, o);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    store_vec<DPL>(L.fr_kv + e * L.W + d0, kvs[e]);
    store_vec<DPL>(L.fr_sc + e * L.W + d0, scs[e]);
    store_vec<DPL>(L.fr_kv + e * L.W + L.D + d0, kv[e + 4]);
    store_vec<DPL>(L.fr_sc + e * L.W + L.D + d0, sc[e + 4]);
  }
}

// Ratio-4 window boundary on one workgroup of SA + 1 waves: SA attention
// waves (DPLA dims per lane) and one indexer wave (DPLI per lane) pool and
// shift their dims in one pass of loads, then finish the row (the attention
// row's sum of squares meets in LDS).  The frontier and norm pointers and
// dims = D_attn | D_index << 16 (0 without an indexer lane) arrive
// preloaded in scalar registers, so the frontier loads issue at once; the
// rest of the token's arguments (row outputs, position, constants) is read
// from `a` meanwhile.
template <int SA, int DPLA, int DPLI>
__global__ void __launch_bounds__(64 * (SA + 1))
    decode_r4_finish_kernel(float* kv0, float* sc0, float* kv1, float* sc1, const float* nw0, const float* nw1,
                            unsigned dims, DecodeArgs a) {
  __shared__ float s_ss[SA];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave), lane = threadIdx.x % kWave;
  const bool att = wave < SA;
  const int d_idx = (int)(dims >> 16);
  LaneDev L{};  // the fields the pool and the finish read
  L.fr_kv = att ? kv0 : kv1;
  L.fr_sc = att ? sc0 : sc1;
  L.D = att ? (int)(dims & 0xffffu) : d_idx;
  L.W = 2 * L.D;
  L.is_index = att ? 0 : 1;
  if (att) {
    const int d0 = wave * (kWave * DPLA) + lane * DPLA;
    const int64_t k = a.pos / 4;
    float nw[DPLA], o[DPLA];
    load_vec<DPLA>(nw, nw0 + d0);
    RowConsts<DPLA> rc;
    r4_pool_and_shift<DPLA>(L, d0, o, [&] { rc = row_consts<DPLA>(d0, L.D, a.n_rot, a.log2_base, k, 4); });
    const float ss = wave_sum(row_sumsq<DPLA>(o));
    if (lane == 0) s_ss[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int w = 0; w < SA; ++w) tot += s_ss[w];
    finish_row_part<DPLA>(o, nw, L, rms_inv(tot, L.D, a.rms_eps), d0, a.n_rot, rc, a.lane[0].prequant,
                          a.lane[0].rows + k * L.D, lane);
  } else {
    const int64_t k = a.pos / 4;
    float nw[DPLI], o[DPLI];
    RowConsts<DPLI> rc;
    if (d_idx > 0) {
      load_vec<DPLI>(nw, nw1 + lane * DPLI);
      r4_pool_and_shift<DPLI>(L, lane * DPLI, o,
                              [&] { rc = row_consts<DPLI>(lane * DPLI, L.D, a.n_rot, a.log2_base, k, 4); });
    }
    __syncthreads();
    if (d_idx > 0)
      finish_row_wave<DPLI>(o, nw, L, a.n_rot, a.rms_eps, rc, a.lane[1].prequant, a.lane[1].rows + k * L.D, lane);
  }
}

// Ratio-128 window boundary, step 1 of 2: D/32 workgroups of eight row
// groups each pool the frontier's 128 rows for 32 dims.  Thread t takes dim
// 32b + t%32 and rows 16(t/32) .. 16(t/32)+15, all loads issued together;
// the row groups' (max, sum, weighted sum) partials merge in LDS, and the
// pooled value (not yet normalised) goes to the output row, which step 2
// finishes in place.  Spreading the 128 rows over D/32 CUs keeps the step at
// about one memory round trip.
constexpr int kR128Dims = 32, kR128Groups = 8, kR128Rows = 16;
static_assert(kR128Groups * kR128Rows == 128, "row groups cover a window");

__global__ void __launch_bounds__(kR128Dims * kR128Groups) decode_r128_pool_kernel(DecodeArgs a) {
  __shared__ float s_m[kR128Groups][kR128Dims], s_s[kR128Groups][kR128Dims], s_a[kR128Groups][kR128Dims];
  const LaneDev& L = a.lane[0];
  const int t = threadIdx.x, dl = t % kR128Dims, g = t / kR128Dims;
  const int d = blockIdx.x * kR128Dims + dl;
  float kv[kR128Rows][1], sc[kR128Rows][1];
#pragma unroll
  for (int e = 0; e < kR128Rows; ++e) {
    kv[e][0] = L.fr_kv[(g * kR128Rows + e) * L.W + d];
    sc[e][0] = L.fr_sc[(g * kR128Rows + e) * L.W + d];
  }
  float m = sc[0][0];
#pragma unroll
  for (int e = 1; e < kR128Rows; ++e) m = fmaxf(m, sc[e][0]);
  float den = 0.f, num = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int e = 0; e < kR128Rows; ++e) {
      const float w = pool_exp(sc[e][0] - m);
      den += w;
      num = fmaf(w, kv[e][0], num);
    }
  }
  s_m[g][dl] = m;
  s_s[g][dl] = den;
  s_a[g][dl] = num;
  __syncthreads();
  if (t >= kR128Dims) return;
  float M = -INFINITY;
#pragma unroll
  for (int h = 0; h < kR128Groups; ++h) M = fmaxf(M, s_m[h][dl]);
  float D = 0.f, A = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int h = 0; h < kR128Groups; ++h) {
      const float mh = s_m[h][dl];
      const float f = mh == -INFINITY ? 0.f : pool_exp(mh - M);
      D = fmaf(s_s[h][dl], f, D);
      A = fmaf(s_a[h][dl], f, A);
    }
  }
  L.rows[(a.pos / 128) * L.D + d] = D > 0.f ? A / D : 0.f;
}

// Ratio-128 window boundary, step 2 of 2: one wave reads the pooled row back
// and finishes it (norm, tail RoPE, FP8 round trip) in place.  Every store
// depends on the row's sum of squares, so all reads precede all writes.
template <int DPL>
__global__ void __launch_bounds__(kWave) decode_r128_finish_kernel(DecodeArgs a) {
  const LaneDev& L = a.lane[0];
  const int lane = threadIdx.x;
  const int64_t k = a.pos / 128;
  float* row = L.rows + k * L.D;
  float nw[DPL], o[DPL];
  load_vec<DPL>(nw, L.norm_w + lane * DPL);
  load_vec<DPL>(o, row + lane * DPL);
  __builtin_amdgcn_sched_barrier(0);
  const RowConsts<DPL> rc = row_consts<DPL>(lane * DPL, L.D, a.n_rot, a.log2_base, k, 128);  // while the row loads
  __builtin_amdgcn_sched_barrier(0);
  finish_row_wave<DPL>(o, nw, L, a.n_rot, a.rms_eps, rc, L.prequant, row, lane);
}

template <int SA, int DPLA>
void launch_r4_fin(const DecodeArgs& a, int dpli, hipStream_t s, const Timing& tm) {
  const dim3 g(1), b(64 * (SA + 1));
  const LaneDev& A = a.lane[0];
  const bool idx = a.n_lanes > 1;
  const LaneDev& I = a.lane[idx ? 1 : 0];
  const unsigned dims = (unsigned)A.D | (idx ? (unsigned)I.D << 16 : 0u);
#define DS4C_R4FIN(P)                                                                                          \
  hipExtLaunchKernelGGL((decode_r4_finish_kernel<SA, DPLA, P>), g, b, 0, s, tm.start, tm.stop, 0, A.fr_kv, A.fr_sc, \
                        I.fr_kv, I.fr_sc, A.norm_w, I.norm_w, dims, a)
  switch (dpli) {
    case 1: DS4C_R4FIN(1); break;
    case 2: DS4C_R4FIN(2); break;
    case 4: DS4C_R4FIN(4); break;
    default: DS4C_R4FIN(8); break;
  }
#undef DS4C_R4FIN
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int in_dtype, hipStream_t stream, const Timing& tm,
                         const Timing& tm_pool) {
  const bool boundary = (a.pos + 1) % a.ratio == 0;
  const unsigned grid = (unsigned)((a.N + kColsPerBlock - 1) / kColsPerBlock);
  // The packed argument holds K/64 in 10 bits and each block's first
  // column/64 in 7 bits (K and the block sizes are multiples of 64).  Layers
  // that pass the descriptor checks (hidden <= 16384, head_dim <= 512, so
  // N <= 4096) are always inside these limits; this is a guard only.
  if (a.K % 64 || a.K / 64 > 1023 || a.N % 64 || a.N / 64 > 127) return hipErrorInvalidValue;
  GemvLaunch g{};
  g.x = a.x;
  const int pr = (int)(a.pos % a.ratio), slot = (a.ratio == 4 ? 4 : 0) + pr;
  unsigned c[4] = {0u, (unsigned)a.N, (unsigned)a.N, (unsigned)a.N};  // unused blocks start at N
  const float* ape[2] = {nullptr, nullptr};
  for (int s = 0; s < 4; ++s) {
    if (s >= a.n_seg) {  // unused block: never selected
      g.w[s] = a.seg[0].w;
      continue;
    }
    const LaneDev& L = a.lane[s >> 1];
    g.w[s] = a.seg[s].w;
    c[s] = (unsigned)a.seg[s].col0;
    g.st.dst[s] = ((s & 1) ? L.fr_sc : L.fr_kv) + (int64_t)slot * L.W;
    if (s & 1) ape[s >> 1] = L.ape + (int64_t)pr * L.W;
  }
  g.kc = (unsigned)a.K / 64 | c[1] / 64 << 10 | c[2] / 64 << 17 | c[3] / 64 << 24;
  g.ape_a = ape[0];
  g.st.ape_i = ape[1];
  if (ape[1]) {
    const int64_t off = ape[1] - ape[0];
    g.far = off < INT_MIN || off > INT_MAX;
    g.ape_i_off = g.far ? 0 : (int)off;
  }
  if (in_dtype == 1)
    launch_gemv<uint16_t>(g, a.K, grid, stream, tm.start, tm.stop);
  else
    launch_gemv<float>(g, a.K, grid, stream, tm.start, tm.stop);
  if (boundary) {
    if (a.ratio == 4) {
      // Attention rows split over waves as in prefill: two waves of 256 dims
      // at D = 512 (6 % faster than four of 128 for this one-workgroup
      // launch), 128 dims at D = 128 / 256, 64 at D = 64.
      const int dpli = a.n_lanes > 1 ? a.lane[1].D / 64 : 1;
      switch (a.lane[0].D) {
        case 64: launch_r4_fin<1, 1>(a, dpli, stream, tm_pool); break;
        case 128: launch_r4_fin<1, 2>(a, dpli, stream, tm_pool); break;
        case 256: launch_r4_fin<2, 2>(a, dpli, stream, tm_pool); break;
        default: launch_r4_fin<2, 4>(a, dpli, stream, tm_pool); break;
      }
    } else {
      hipExtLaunchKernelGGL(decode_r128_pool_kernel, dim3(a.lane[0].D / kR128Dims), dim3(kR128Dims * kR128Groups), 0,
                            stream, tm_pool.start, nullptr, 0, a);
      const dim3 g(1), b(kWave);
      switch (a.lane[0].D / 64) {
        case 1: hipExtLaunchKernelGGL((decode_r128_finish_kernel<1>), g, b, 0, stream, nullptr, tm_pool.stop, 0, a); break;
        case 2: hipExtLaunchKernelGGL((decode_r128_finish_kernel<2>), g, b, 0, stream, nullptr, tm_pool.stop, 0, a); break;
        case 4: hipExtLaunchKernelGGL((decode_r128_finish_kernel<4>), g, b, 0, stream, nullptr, tm_pool.stop, 0, a); break;
        default: hipExtLaunchKernelGGL((decode_r128_finish_kernel<8>), g, b, 0, stream, nullptr, tm_pool.stop, 0, a); break;
      }
    }
  }
  return hipGetLastError();
}

}  // namespace ds4c
