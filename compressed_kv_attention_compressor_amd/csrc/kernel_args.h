// Kernel argument blocks, filled on the host and passed by value.
#pragma once

#include <stdint.h>

namespace ds4c {

// One compressor lane as the kernels see it.
struct LaneDev {
  const float* ape;     // [ratio, W]
  const float* norm_w;  // [D]
  float* rows;          // [cap, D]; row k of the lane goes to rows + k*D
  float* prequant;      // nullable [n_emit, D]; row k goes to prequant + (k - k_lo)*D
  float* fr_kv;         // frontier kv    [coff*ratio, W]
  float* fr_sc;         // frontier score [coff*ratio, W]
  int D;                // head_dim
  int W;                // coff * D
  int kv_col;           // column of the lane's kv block in a projection row
  int sc_col;           // column of the lane's score block in a projection row
  int is_index;         // 0: attention (FP8), 1: indexer (Hadamard + FP4)
};

// A block of output columns [col0, col0 + n) computed from weights w [n, K].
struct ProjSeg {
  const void* w;
  int col0;
  int n;
};

struct ProjArgs {
  const void* x;        // [M, K] row-major, bf16 or f32
  float* out;           // [M, N] row-major f32
  int64_t M;
  int K;
  int N;
  int n_seg;
  ProjSeg seg[4];
};

struct PoolArgs {
  const float* proj;    // [T, ld] projection workspace (scores without APE)
  int64_t ld;
  int64_t n0;           // tokens before this call
  int64_t T;            // tokens in this call
  int64_t k_lo, k_hi;   // rows emitted: windows k_lo .. k_hi-1
  int n_head;           // leading windows that read the incoming frontier
  int ratio;
  int n_rot;
  int n_lanes;
  double log2_base;     // log2 of the compression RoPE base
  float rms_eps;
  LaneDev lane[2];
  float* part;          // ratio 128: [k_hi-k_lo][2 halves][max, sum, weighted sum][D]
};

struct DecodeArgs {
  const void* x;        // [K]
  int K;
  int N;
  int n_seg;
  ProjSeg seg[4];
  int seg_lane[4];      // lane index of each segment
  int seg_score[4];     // 1 if the segment holds scores, 0 if kv
  int64_t pos;
  int ratio;
  int n_rot;
  int n_lanes;
  double log2_base;
  float rms_eps;
  LaneDev lane[2];
};

struct FillArgs {
  float* kv[2];
  float* sc[2];
  int64_t n[2];         // floats per tensor
  unsigned* ctrl;       // control block words
  int n_ctrl;
  int n_lanes;
};

}  // namespace ds4c
