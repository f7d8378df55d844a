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

// Ratio-4 window pool fused into the projection epilogue (calls that start
// on a window boundary).  Output column tile tn holds dims 40*tn .. 40*tn+39
// of the concatenated lanes (attention dims, then indexer dims) as four runs
// of 40 columns: kv of the previous half, kv of the current half, score of
// the previous half, score of the current half.  Call-relative token t is
// tile row t; window j pools tokens 4j-4 .. 4j-1 (previous half) and
// 4j .. 4j+3 (current half).
struct FuseArgs {
  int on;               // 0: plain [M, N] output in ProjArgs::out
  int ratio;            // 4: layout above; 128: tile tn holds dims 64*tn .. 64*tn+63 as
                        // [kv (64) | score (64)] and tile row t is call-relative token t
  int d_attn, d_idx;    // head dims (d_idx = 0 without an indexer lane)
  int d_tot;            // d_attn + d_idx: columns of o and part
  int W[2];             // lane widths (2 * head dim)
  int n_orig;           // columns of a staged token (the plain layout)
  int64_t n_emit;       // windows the call emits
  int64_t carry_lo;     // first call-relative token the frontier keeps
  const float* ape[2];  // [4, W] per lane
  float* o;             // [n_emit, d_tot]: pooled rows (before the norm) of windows j % 64 != 0
  float* part;          // [M tiles][2 halves][max, sum, weighted sum][d_tot] of windows j % 64 == 0
  float* stage;         // [T - carry_lo, n_orig]: kv and score + APE of the kept tokens
  const float* fr_kv[2];  // incoming frontier rows 0..3 hold window 0's previous half
  const float* fr_sc[2];
};

struct ProjArgs {
  const void* x;        // [M, K] row-major, bf16 or f32
  float* out;           // [M, N] row-major f32 (unfused); with a K split, plane s of
                        // k_split planes at out + s * split_stride holds the sum over
                        // K columns [s * k_len, (s + 1) * k_len)
  int64_t M;
  int K;
  int N;
  int k_split;          // 1, or the number of K ranges (plain 64x64 / 128x128 kernel only)
  int k_len;            // K / k_split, a multiple of 64
  int64_t split_stride; // floats between output planes (M * N)
  int n_seg;
  ProjSeg seg[4];       // attention wkv, wgate, then indexer wkv, wgate
  FuseArgs fuse;
};

struct PoolArgs {
  const float* proj;    // [T, ld] projection workspace (scores without APE)
  int64_t ld;
  int64_t n0;           // tokens before this call
  int64_t T;            // tokens in this call
  int64_t k_lo, k_hi;   // rows emitted: windows k_lo .. k_hi-1
  int ratio;
  int n_rot;
  int n_lanes;
  double log2_base;     // log2 of the compression RoPE base
  float rms_eps;
  LaneDev lane[2];
  float* part;          // ratio 128: [k_hi-k_lo][2 halves][max, sum, weighted sum][D];
                        // fused ratio 4: FuseArgs::part
  // Fused ratio 4 (n0 % 4 == 0): the finisher reads these instead of proj.
  const float* o;       // FuseArgs::o
  const float* stage;   // FuseArgs::stage
  int d_tot;
  int64_t carry_lo;
};

// The decode GEMV's arguments.  What a workgroup needs before its loads is
// passed as leading scalar kernel arguments, which the dispatch preloads
// into scalar registers (no argument load from memory before the weight
// loads); the frontier rows the results go to are read from this struct
// while the weights stream.  The token's column blocks are resolved on the
// host (blocks are ordered attention kv, attention score, indexer kv,
// indexer score).
struct GemvStore {
  float* dst[4];        // frontier row (coff-1)*ratio + pos%ratio, at the block's first dim
  const float* ape_i;   // indexer lane's APE row, used when it is not within 2^31 floats of the attention lane's
};

struct DecodeArgs {
  const void* x;        // [K]
  int K;
  int N;
  int n_seg;
  ProjSeg seg[4];
  int64_t pos;
  int ratio;
  int n_rot;
  int n_lanes;
  double log2_base;
  float rms_eps;
  LaneDev lane[2];
};

// Indexer scoring and top-k of one query token.
struct IndexerArgs {
  const float* q;       // [H, Dh] query heads (before the QAT round trip)
  const float* head_w;  // [H] head weights
  const float* rows;    // [n, Dh] compressed indexer rows (rotated, QAT applied)
  int64_t n;            // rows
  int H;                // heads, a multiple of 4, <= 64
  int Dh;               // 64 or 128
  float* scores;        // [n] every row's score
  float* q_hat;         // nullable [H, Dh]: the query after the round trip
  int32_t* out_idx;     // [min(n, k)] selected rows, descending score
  float* out_score;     // [min(n, k)] their scores
  int k;                // 1 .. 512
  uint64_t* cand;       // [n_chunks * k] sort keys surviving each chunk
  uint32_t* hist;       // [ceil(n / 64), 64] per 64-row block: how many of its rows' keys have each top
                        // byte, bins 4i .. 4i+3 in the bytes (low first) of word i
  int n_chunks;         // ceil(n / kIndexerChunk)
};

struct MixedAttnArgs {
  const float* q;        // [H, D] query heads
  const float* ring;     // [ring_cap, D] raw sliding-window rows, position p at row p % ring_cap
  const float* comp;     // [n_comp, D] compressed attention rows
  const int32_t* topk;   // [k] selected compressed rows (negative: skipped)
  float* part_o;         // [n_split, H, D] weighted rows per split (workspace)
  float* part_m;         // [n_split, H] max logit per split
  float* part_l;         // [n_split, H] softmax sum per split
  float* out;            // [H, D]
  int H;                 // heads, a multiple of 8
  int D;                 // 64, 128, 256 or 512
  int ring_cap;
  int ring_row0;         // ring row of the first attended raw position
  int k;
  int n_split;
  int n_raw;             // attended raw rows, ring rows ring_row0 .. ring_row0 + n_raw - 1 (wrapped)
  int64_t visible;       // compressed rows visible to the query
  float scale;           // 1 / sqrt(D)
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
