// Device helpers shared by the compressor kernels (gfx950, wave64).
//
// The row epilogue (RMS norm, tail RoPE, FP8 or Hadamard+FP4 round trip)
// runs on one wavefront holding one D-wide row, DPL = D/64 consecutive dims
// per lane.  Reductions over the row or over a codec block are xor-butterfly
// exchanges (lane_xor), so every lane ends with bitwise the same value.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernel_args.h"

namespace ds4c {

constexpr int kWave = 64;

// The value that lane (lane ^ m) holds, for the whole wave (every lane
// active).  Once loops are unrolled m is a constant and the switch folds:
// distances 1 and 2 are DPP quad permutes; 4 and 8 two DPP mirrors each
// (the half-row mirror is lane ^ 7, the row mirror lane ^ 15, so ^7 then ^3
// gives ^4 and ^15 then ^7 gives ^8); 16 and 32 are the row-pair and
// half-wave swaps (v_permlane16_swap / v_permlane32_swap, with the source
// itself as both operands: a lane in the upper row or half reads the first
// result, a lane in the lower one the second).  All of these are VALU
// operations; a general distance falls back to the LDS permute.
template <int CTRL>
__device__ __forceinline__ int dpp_mov(int v) {
  return __builtin_amdgcn_mov_dpp(v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ int lane_xor(int v, int m) {
  switch (m) {
    case 1: return dpp_mov<0xB1>(v);                  // quad_perm [1,0,3,2]
    case 2: return dpp_mov<0x4E>(v);                  // quad_perm [2,3,0,1]
    case 4: return dpp_mov<0x1B>(dpp_mov<0x141>(v));  // half-row mirror, quad_perm [3,2,1,0]
    case 8: return dpp_mov<0x141>(dpp_mov<0x140>(v));  // row mirror, half-row mirror
    case 16: {
      const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
      return (__lane_id() & 16) ? r[0] : r[1];
    }
    case 32: {
      const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
      return (__lane_id() & 32) ? r[0] : r[1];
    }
    default: return __shfl_xor(v, m, kWave);
  }
}
__device__ __forceinline__ float lane_xor(float v, int m) {
  return __builtin_bit_cast(float, lane_xor(__builtin_bit_cast(int, v), m));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += lane_xor(v, o);
  return v;
}

// Maximum over aligned groups of G lanes (G a power of two <= 64).
template <int G>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = G / 2; o > 0; o >>= 1) v = fmaxf(v, lane_xor(v, o));
  return v;
}

// ---------------------------------------------------------------------------
// Block scales and element rounding (Part 3 §9 names E4M3 and FP4; the
// formats are the OCP E4M3 "fn" and E2M1 element types).
//
// A block is scaled by 2^k with the smallest integer k for which its largest
// magnitude fits the format's largest finite value, so nothing saturates.
// frexpf gives amax = f * 2^e with f in [0.5, 1); the largest finite value
// is 448 = 0.875 * 2^9 for E4M3 and 6 = 0.75 * 2^3 for E2M1.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int e4m3_block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  float f = frexpf(amax, &e);
  return f <= 0.875f ? e - 9 : e - 8;
}

__device__ __forceinline__ int e2m1_block_exp(float amax) {
  if (!(amax > 0.f)) return 0;
  int e;
  float f = frexpf(amax, &e);
  return f <= 0.75f ? e - 3 : e - 2;
}

// Nearest value of a (sign, exponent, mantissa) grid, ties to even, for
// |v| within the grid's finite range.  Between 2^E and 2^(E+1) the grid step
// is 2^(E - mbits); below the smallest normal 2^emin the step is
// 2^(emin - mbits).  Scaling by the step is exact, rintf rounds half to even
// (even integer == even mantissa), and scaling back is exact.
template <int MBITS, int EMIN>
__device__ __forceinline__ float round_to_grid(float v) {
  float a = fabsf(v);
  int e;
  frexpf(a, &e);  // a in [2^(e-1), 2^e)
  int q = max(e - 1, EMIN) - MBITS;
  float r = rintf(ldexpf(a, -q));
  return copysignf(ldexpf(r, q), v);
}

__device__ __forceinline__ float rne_e4m3(float v) { return round_to_grid<3, -6>(v); }
__device__ __forceinline__ float rne_e2m1(float v) { return round_to_grid<1, 0>(v); }

// Vector load/store of DPL consecutive floats (DPL in {1, 2, 4, 8}); the
// address is DPL*4-byte aligned (16-byte for DPL >= 4).
template <int DPL>
__device__ __forceinline__ void load_vec(float (&v)[DPL], const float* __restrict__ p) {
  if constexpr (DPL == 1) {
    v[0] = p[0];
  } else if constexpr (DPL == 2) {
    float2 t = *reinterpret_cast<const float2*>(p);
    v[0] = t.x; v[1] = t.y;
  } else {
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
      float4 t = *reinterpret_cast<const float4*>(p + i);
      v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
    }
  }
}

// The same load with the nontemporal hint, for data read exactly once (the
// projection rows a plain pool consumes).
template <int DPL>
__device__ __forceinline__ void load_vec_stream(float (&v)[DPL], const float* __restrict__ p) {
  if constexpr (DPL == 1) {
    v[0] = __builtin_nontemporal_load(p);
  } else if constexpr (DPL == 2) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 t = __builtin_nontemporal_load(reinterpret_cast<const f2*>(p));
    v[0] = t.x; v[1] = t.y;
  } else {
    typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < DPL; i += 4) {
      const f4 t = __builtin_nontemporal_load(reinterpret_cast<const f4*>(p + i));
      v[i] = t.x; v[i + 1] = t.y; v[i + 2] = t.z; v[i + 3] = t.w;
    }
  }
}

template <int DPL>
__device__ __forceinline__ void store_vec(float* __restrict__ p, const float (&v)[DPL]) {
  if constexpr (DPL == 1) {
    p[0] = v[0];
  } else if constexpr (DPL == 2) {
    *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
  } else {
#pragma unroll
    for (int i = 0; i < DPL; i += 4)
      *reinterpret_cast<float4*>(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  }
}

// sin and cos of 2*pi*t for |t| <= 1/2 (t in turns).  Quadrant q = rint(4t)
// leaves r = 2*pi*(t - q/4) in [-pi/4, pi/4], where the Taylor series of sin
// (to r^9) and cos (to r^8) are within 2e-9 of the true values; the quadrant
// then swaps and negates them.
__device__ __forceinline__ void sincos_turns(float t, float* s, float* c) {
  const float q = rintf(4.0f * t);
  const float r = (t - 0.25f * q) * 6.28318530717958647692f;
  const float r2 = r * r;
  const float sr = r * (1.0f + r2 * (-1.0f / 6 + r2 * (1.0f / 120 + r2 * (-1.0f / 5040 + r2 * (1.0f / 362880)))));
  const float cr = 1.0f + r2 * (-0.5f + r2 * (1.0f / 24 + r2 * (-1.0f / 720 + r2 * (1.0f / 40320))));
  const int qi = ((int)q) & 3;
  *s = qi == 0 ? sr : qi == 1 ? cr : qi == 2 ? -sr : -cr;
  *c = qi == 0 ? cr : qi == 1 ? -sr : qi == 2 ? -cr : sr;
}

// RoPE angle of pair i at position pos: pos * base^(-2i/n_rot) radians.  It
// is formed in fp64 (positions reach 10^5 and beyond, where a float angle
// would be off by more than 10^-3 rad) as a number of turns, whose fractional
// part then goes to the float sin/cos above.
__device__ __forceinline__ void rope_sincos(double pos, int i, int n_rot, double log2_base, float* s,
                                            float* c) {
  const double theta = exp2(-2.0 * (double)i / (double)n_rot * log2_base);
  const double turns = pos * theta * 0.15915494309189533577;  // 1 / (2 pi)
  sincos_turns((float)(turns - rint(turns)), s, c);
}

// Softmax weight e^x for x <= 0: 2^(x log2 e) through the hardware base-2
// exponential.  Rounding x log2 e costs a relative error of at most
// |x| * 2^-24 * ln 2 in the result (below 1e-6 for |x| < 20; weights of
// entries further below the maximum are under 2e-9) plus the instruction's
// own error of about one ulp; e^-inf = 0.
__device__ __forceinline__ float pool_exp(float x) { return __builtin_amdgcn_exp2f(x * 1.44269504088896341f); }

// Softmax pool of E entries per dim: o = sum w*kv / sum w, w = exp(s - max).
template <int E, int DPL>
__device__ __forceinline__ void pool_entries(const float (&kv)[E][DPL], const float (&sc)[E][DPL], float (&o)[DPL]) {
#pragma unroll
  for (int i = 0; i < DPL; ++i) {
    float m = sc[0][i];
#pragma unroll
    for (int e = 1; e < E; ++e) m = fmaxf(m, sc[e][i]);
    float den = 0.f, num = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float w = pool_exp(sc[e][i] - m);
        den += w;
        num = fmaf(w, kv[e][i], num);
      }
    }
    o[i] = den > 0.f ? num / den : 0.f;
  }
}

// ---------------------------------------------------------------------------
// Row epilogue.  A row of D dims is held by one or more waves; this lane
// holds dims d0 .. d0+DPL-1.  `inv` is 1/sqrt(mean(o^2) + eps) of the whole
// row.  Applies the norm weight, tail RoPE (Part 3 §8), writes the pre-codec
// row if asked, then the lane codec (Part 3 §9), and writes the final row.
// FP8 blocks (64 dims) must lie within one wave; the indexer's Hadamard
// rotation needs the whole row in one wave (D == 64 * DPL).
// ---------------------------------------------------------------------------
template <int DPL>
__device__ __forceinline__ float row_sumsq(const float (&y)[DPL]) {
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < DPL; ++i) ss = fmaf(y[i], y[i], ss);
  return ss;
}

// Indexer QAT round trip of NB independent D-wide rows, each held by LANES
// consecutive lanes of one wave (D == LANES * DPL; the lane at position c of
// its group holds dims c*DPL .. of each of its rows): the orthonormal
// Walsh-Hadamard rotation (Sylvester order; butterflies (a, b) -> (a + b,
// a - b) on index pairs (j, j + h) for h = 1, 2, 4, ...; strides below DPL
// inside a lane, the rest across lanes), scaled by 1/sqrt(D), then FP4 E2M1
// in blocks of 32 dims (32/DPL lanes) with the power-of-two block scale.  The
// rows stay rotated.  Every stage runs over all NB rows before the next, so
// the rows' cross-lane exchanges overlap.  Across lanes the butterfly is one
// fma with a weight of +1 (lower lane: b + a) or -1 (upper lane: a - b),
// exact in the product, so each output is the same single rounding of a + b
// or a - b as inside a lane.
template <int DPL, int NB, int LANES = kWave>
__device__ __forceinline__ void hadamard_fp4_rows(float (&y)[NB][DPL], float scale, int lane) {
  static_assert(LANES >= 1 && LANES <= kWave && (LANES & (LANES - 1)) == 0, "lanes per row");
#pragma unroll
  for (int h = 1; h < DPL; h <<= 1) {
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int i = 0; i < DPL; ++i) {
        if ((i & h) == 0) {
          const float a = y[n][i], b = y[n][i + h];
          y[n][i] = a + b;
          y[n][i + h] = a - b;
        }
      }
    }
  }
#pragma unroll
  for (int m = 1; m < LANES; m <<= 1) {
    const float sgn = (lane & m) ? -1.f : 1.f;
#pragma unroll
    for (int n = 0; n < NB; ++n) {
#pragma unroll
      for (int i = 0; i < DPL; ++i) y[n][i] = fmaf(sgn, y[n][i], lane_xor(y[n][i], m));
    }
  }
  float amax[NB];
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    amax[n] = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) {
      y[n][i] *= scale;
      amax[n] = fmaxf(amax[n], fabsf(y[n][i]));
    }
  }
#pragma unroll
  for (int o = 32 / DPL / 2; o > 0; o >>= 1)
#pragma unroll
    for (int n = 0; n < NB; ++n) amax[n] = fmaxf(amax[n], lane_xor(amax[n], o));
#pragma unroll
  for (int n = 0; n < NB; ++n) {
    const int kexp = e2m1_block_exp(amax[n]);
#pragma unroll
    for (int i = 0; i < DPL; ++i) y[n][i] = ldexpf(rne_e2m1(ldexpf(y[n][i], -kexp)), kexp);
  }
}

template <int DPL>
__device__ __forceinline__ void hadamard_fp4(float (&y)[DPL], float scale, int lane) {
  hadamard_fp4_rows<DPL, 1>(*reinterpret_cast<float (*)[1][DPL]>(&y), scale, lane);
}

// The rotation's scale 1/sqrt(D), rounded once to float.
__device__ __forceinline__ float hadamard_scale(int D) { return (float)(1.0 / sqrt((double)D)); }

// Per-row constants of the finish that need none of the row's data: the RoPE
// sin/cos of the pairs this lane rotates (with DPL >= 2, pairs (d0 + 2p,
// d0 + 2p + 1) for p < DPL/2; with DPL == 1, the pair of dim d0 and its
// neighbouring lane) and the indexer rotation's scale.  They depend on the
// position and the dims only, so a caller computes them between issuing its
// loads and using the data, where the fp64 arithmetic overlaps the memory
// round trip.  Every lane computes them (a lane outside the tail takes pair
// 0 and never uses it).
template <int DPL>
struct RowConsts {
  static constexpr int kPairs = DPL >= 2 ? DPL / 2 : 1;
  float s[kPairs], c[kPairs];
  float hscale;
};
template <int DPL>
__device__ __forceinline__ RowConsts<DPL> row_consts(int d0, int D, int n_rot, double log2_base, int64_t k,
                                                     int ratio) {
  RowConsts<DPL> r;
  const int n_nope = D - n_rot;
  const double pos = (double)k * (double)ratio;
#pragma unroll
  for (int p = 0; p < RowConsts<DPL>::kPairs; ++p) {
    const int i = (DPL >= 2 ? d0 + 2 * p - n_nope : d0 - n_nope) >> 1;
    rope_sincos(pos, i > 0 ? i : 0, n_rot, log2_base, &r.s[p], &r.c[p]);
    // An empty asm that takes the values keeps the compiler from sinking
    // their computation to the later point of use.
    asm volatile("" : "+v"(r.s[p]), "+v"(r.c[p]));
  }
  r.hscale = hadamard_scale(D);
  asm volatile("" : "+v"(r.hscale));
  return r;
}

// w holds the norm weights of this lane's dims, loaded by the caller ahead
// of the row's entries so that no load sits between the pool and the store;
// rc holds the row's constants (row_consts).
template <int DPL>
__device__ __forceinline__ void finish_row_part(float (&y)[DPL], const float (&w)[DPL], const LaneDev& L, float inv,
                                                int d0, int n_rot, const RowConsts<DPL>& rc,
                                                float* __restrict__ prequant_row, float* __restrict__ out_row,
                                                int lane) {
  const int D = L.D;
#pragma unroll
  for (int i = 0; i < DPL; ++i) y[i] = y[i] * w[i] * inv;

  // Tail RoPE: the last n_rot dims, adjacent pairs (2i, 2i+1), rotated by
  // (k * ratio) * base^(-2i/n_rot) radians.
  const int n_nope = D - n_rot;
  if constexpr (DPL >= 2) {
    if (d0 >= n_nope) {
#pragma unroll
      for (int i = 0; i < DPL; i += 2) {
        const float sf = rc.s[i / 2], cf = rc.c[i / 2];
        const float a = y[i], b = y[i + 1];
        y[i] = a * cf - b * sf;
        y[i + 1] = a * sf + b * cf;
      }
    }
  } else {
    // One dim per lane: the pair partner is the neighbouring lane.
    const float other = lane_xor(y[0], 1);
    if (d0 >= n_nope) {
      const float sf = rc.s[0], cf = rc.c[0];
      if ((lane & 1) == 0)
        y[0] = y[0] * cf - other * sf;  // a' = a cos - b sin
      else
        y[0] = other * sf + y[0] * cf;  // b' = a sin + b cos
    }
  }

  if (prequant_row) store_vec<DPL>(prequant_row + d0, y);

  if (!L.is_index) {
    // FP8 E4M3 round trip on dims [0, n_nope) in blocks of 64 (64/DPL lanes).
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < DPL; ++i) amax = fmaxf(amax, fabsf(y[i]));
    amax = group_max<kWave / DPL>(amax);
    if (d0 < n_nope) {
      const int kexp = e4m3_block_exp(amax);
#pragma unroll
      for (int i = 0; i < DPL; ++i) y[i] = ldexpf(rne_e4m3(ldexpf(y[i], -kexp)), kexp);
    }
  } else {
    hadamard_fp4<DPL>(y, rc.hscale, lane);
  }

  store_vec<DPL>(out_row + d0, y);
}

__device__ __forceinline__ float rms_inv(float sumsq, int D, float eps) {
  return 1.0f / sqrtf(sumsq / (float)D + eps);
}

// Whole row in one wave (D == 64 * DPL).
template <int DPL>
__device__ __forceinline__ void finish_row_wave(float (&y)[DPL], const float (&w)[DPL], const LaneDev& L, int n_rot,
                                                float rms_eps, const RowConsts<DPL>& rc, float* __restrict__ prequant_row,
                                                float* __restrict__ out_row, int lane) {
  const float inv = rms_inv(wave_sum(row_sumsq<DPL>(y)), L.D, rms_eps);
  finish_row_part<DPL>(y, w, L, inv, lane * DPL, n_rot, rc, prequant_row, out_row, lane);
}

}  // namespace ds4c
