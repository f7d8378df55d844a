/*
 * ds4c — the compressed-KV compressor of the ds4 (DwarfStar) DeepSeek-V4
 * engine, as a C-ABI library for AMD Instinct MI355X (gfx950).
 *
 * Sources of what is computed: Yoshiya Kato's Qiita series on ds4, "Part 3"
 * (Metal グラフと圧縮 KV の実装を読む: compressor、indexer、HC、tail-only
 * RoPE) and "Part 4" (KV キャッシュをディスクの一級市民にする: DwarfStar の
 * KVC と DSV4 ペイロードを読む).  Section numbers below refer to those pages.
 *
 * Per layer and per lane, each token is projected by wkv (kv candidates)
 * and wgate (scores); the learned position bias APE[pos % ratio] is added to
 * the scores; kv and scores go into a small recurrent state (the
 * "frontier"); when a ratio window closes, every output dim is the softmax
 * (over the window's entries) weighted mean of its kv entries; the pooled
 * row is RMS-normalised, its last n_rot dims are rotated (tail RoPE with
 * the compression base), and it goes through the FP8 E4M3 round trip
 * (attention lane, non-RoPE dims) or the Hadamard + FP4 E2M1 round trip
 * (indexer lane).  Part 3 §4, §5, §8, §9.  Beside the compressor, its two
 * consumers on ratio-4 layers: the indexer's top-k over the compressed
 * indexer rows (Part 3 §6) and the indexed mixed attention over the raw
 * window and the selected compressed rows (Part 3 §7).
 *
 * Conventions for every call:
 *   - Pointers are device pointers unless the name starts with host_.
 *   - All device buffers are owned by the caller.  prefill and decode_one
 *     never allocate device memory.
 *   - `stream` is a hipStream_t (NULL = the null stream).  prefill,
 *     decode_one and frontier_init only enqueue work and return; the
 *     frontier's host counters are updated at enqueue (they depend only on
 *     token counts).  save and load synchronise `stream`.
 *   - Every argument is validated on the host before anything is enqueued.
 *     On failure the call returns a negative ds4c_status, enqueues nothing,
 *     writes nothing and leaves the frontier unchanged.
 *   - One frontier must not be used by two calls at once; different
 *     frontiers may be used from different threads.
 *   - prefill, decode_one, frontier_init, the stack prefill/decode calls,
 *     the indexer and the mixed attention enqueue kernel launches only (no
 *     memset or copy nodes), so with kernel timing and cache eviction off
 *     (ds4c_profile_enable(0), no ds4c_profile_evict buffer) they may be
 *     recorded under HIP stream capture.  A captured sequence replays at the
 *     positions and buffers it was recorded with: the host counters advance
 *     at capture, not at replay, so before each replay the caller puts the
 *     frontier's device state back where it stood at capture.
 *   - Little-endian hosts only (the frontier blob is little-endian).
 *   - No C++ exception crosses this interface.
 */
#ifndef DS4C_H
#define DS4C_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum ds4c_status {
  DS4C_OK = 0,
  DS4C_EINVAL = -1,  /* null or misaligned pointer, bad ratio/dtype, missing or extra lane */
  DS4C_ESHAPE = -2,  /* a dimension the kernels do not support (see ds4c_layer) */
  DS4C_ECAP = -3,    /* row buffer, workspace or host buffer too small */
  DS4C_EPOS = -4,    /* frontier counters inconsistent with each other */
  DS4C_EFORMAT = -5, /* frontier blob: bad magic, version, shape or length */
  DS4C_EDEVICE = -6  /* a HIP runtime call failed */
} ds4c_status;

typedef enum ds4c_dtype { DS4C_F32 = 0, DS4C_BF16 = 1 } ds4c_dtype;

/* One compressor lane (Part 3 §6 names the per-lane tensors: *_compressor_kv,
 * *_compressor_gate, *_compressor_ape, *_compressor_norm).
 * coff = 2 on ratio-4 layers, 1 on ratio-128 layers (Part 3 §5); W = coff*head_dim. */
typedef struct ds4c_lane {
  int32_t head_dim;     /* D: a power of two, 64 <= D <= 512 (one row per 64-lane wavefront).
                           attention lane: (D - n_rot) % 64 == 0 (whole FP8 blocks). */
  const void *wkv;      /* [W, hidden] row-major, layer in_dtype, 16-byte aligned */
  const void *wgate;    /* [W, hidden] row-major, layer in_dtype, 16-byte aligned */
  const float *ape;     /* [ratio, W] float32, 16-byte aligned */
  const float *norm_w;  /* [D] float32 RMS-norm weight, 16-byte aligned */
} ds4c_lane;

/* One compressed layer.  ratio 4 layers have an attention and an indexer
 * lane; ratio 128 layers only an attention lane (index must be all zero).
 * Uncompressed layers (ratio 0, Part 3 §1) have no compressor: DS4C_EINVAL. */
typedef struct ds4c_layer {
  int32_t ratio;        /* 4 or 128 */
  int32_t hidden;       /* K of the projections: hidden % 64 == 0, <= 16384 */
  int32_t n_rot;        /* RoPE tail width (64 in ds4, Part 3 §8): even, 0 < n_rot <= D */
  int32_t in_dtype;     /* ds4c_dtype of x, wkv and wgate */
  float rope_base;      /* compression RoPE base (> 0): theta_i = base^(-2i/n_rot) */
  float rms_eps;        /* RMS-norm epsilon (>= 0) */
  ds4c_lane attn;       /* rows get the FP8 E4M3 round trip on dims [0, D - n_rot) */
  ds4c_lane index;      /* rows get Hadamard(D)/sqrt(D) then FP4 E2M1, blocks of 32 */
} ds4c_layer;

/* Per-layer compressor state.  The caller owns it and allocates `state`
 * (ds4c_frontier_bytes bytes of device memory, 256-byte aligned); the
 * library keeps the counters.  n_tokens is the absolute position of the next
 * token; n_comp / n_index_comp count the rows appended so far and always
 * equal n_tokens / ratio (0 for the indexer on ratio-128 layers).  Part 3 §2
 * (ds4_layer_cache), Part 4 §7 (frontier tensors). */
typedef struct ds4c_frontier {
  int64_t n_tokens;
  int64_t n_comp;
  int64_t n_index_comp;
  void *state;
} ds4c_frontier;

/* Bytes of device memory a layer's frontier needs (Part 3 §2: the layer
 * cache keeps attn_state_kv / attn_state_score and index_state_kv /
 * index_state_score; Part 3 §5: a ratio-4 lane's state is 8 rows of width
 * 2 * head_dim, a ratio-128 lane's 128 rows of head_dim): a 256-byte block
 * reserved for the library then, per lane, kv and score tensors of
 * [coff*ratio, W] float32.  0 if the layer descriptor is invalid. */
size_t ds4c_frontier_bytes(const ds4c_layer *layer);

/* Bytes of device workspace ds4c_compress_prefill needs for calls of up to
 * max_tokens tokens (Part 3 §4: the kv and score projections of every token
 * of the chunk, pooled per window): the [T, N] float32 projection (N = 2 *
 * sum of lane widths; a short call that splits K over several ranges keeps
 * up to min(1024, 16 T) rows of partial sums, so T rows become max(T,
 * min(1024, 16 T))) plus per-row pooling scratch on ratio-128 layers, or the
 * pooled rows and kept tokens of a call that pools in the projection, if
 * larger.  0 if invalid.  Pure function of its arguments; no device call. */
size_t ds4c_workspace_bytes(const ds4c_layer *layer, int64_t max_tokens);

/* Bytes of the host blob ds4c_frontier_save writes for this layer (Part 4
 * §5-§7: the frontier tensors are saved with the counters so a restored
 * session continues mid-window): the 56-byte header, then each lane's kv and
 * score tensors.  0 if the layer descriptor is invalid. */
size_t ds4c_frontier_blob_bytes(const ds4c_layer *layer);

/* Empty state and counters 0 (Part 3 §4: the pool weighs entries by
 * exp(score - max) and returns 0 when the weights sum to 0, so an empty row
 * is kv 0 with score -inf: it takes no weight, and a window with no token
 * yet pools to 0): every kv 0, every score -inf, the control block 0.
 * Enqueued on `stream` as a fill kernel (no memset).  DS4C_EINVAL for a bad
 * descriptor or frontier (nothing enqueued), DS4C_EDEVICE on a launch
 * failure.  Call it once before a frontier's first use. */
int ds4c_frontier_init(const ds4c_layer *layer, ds4c_frontier *frontier, void *stream);

/* Compress a chunk of T tokens x [T, hidden] (in_dtype, row-major) at
 * absolute positions frontier->n_tokens ... + T - 1 (Part 3 §3: chunks keep
 * windows on absolute positions; the frontier carries partial windows).
 *
 * Appends n_emit = (n0+T)/ratio - n0/ratio rows to each lane (n0 = the
 * frontier's n_tokens): row k (the window of tokens k*ratio ...) is written
 * to attn_rows[k * D_attn ...] and index_rows[k * D_index ...], so rows
 * n_comp .. n_comp+n_emit-1 of the caller's append-only buffers (Part 4 §6).
 * attn_cap / index_cap are the buffers' capacities in rows; index_rows must
 * be NULL with index_cap 0 on ratio-128 layers.
 *
 * attn_prequant / index_prequant (nullable, [n_emit, D]) receive each new
 * row after RMS norm and tail RoPE, before its codec; row 0 is the call's
 * first new row.
 *
 * workspace: device, >= ds4c_workspace_bytes(layer, T) bytes, 256-byte
 * aligned, contents undefined on entry and exit.
 *
 * A call with T == 1 runs the decode step (as ds4c_compress_decode_one, same
 * results; the workspace is still validated but not touched).
 *
 * Errors: DS4C_EINVAL, DS4C_ESHAPE, DS4C_ECAP (rows or workspace),
 * DS4C_EPOS (counters), DS4C_EDEVICE.  T == 0 is a no-op returning DS4C_OK. */
int ds4c_compress_prefill(const ds4c_layer *layer, ds4c_frontier *frontier,
                          const void *x, int64_t T,
                          float *attn_rows, int64_t attn_cap,
                          float *index_rows, int64_t index_cap,
                          void *workspace, size_t ws_bytes,
                          float *attn_prequant, float *index_prequant,
                          void *stream);

/* One decode token x [hidden] at position frontier->n_tokens (Part 3 §4:
 * compressor_decode_one): project, store into frontier row
 * (coff-1)*ratio + pos % ratio with the APE added to the score, and when
 * (pos+1) % ratio == 0 pool the frontier into row pos/ratio of each lane
 * (norm, tail RoPE, codec) and, on ratio-4 layers, copy rows 4..7 to rows
 * 0..3 (Part 3 §5).  Rows and prequant as for prefill (prequant row 0 is
 * the emitted row, if any).  Needs no workspace.  Same errors as prefill. */
int ds4c_compress_decode_one(const ds4c_layer *layer, ds4c_frontier *frontier,
                             const void *x,
                             float *attn_rows, int64_t attn_cap,
                             float *index_rows, int64_t index_cap,
                             float *attn_prequant, float *index_prequant,
                             void *stream);

/* Serialise the frontier into host memory (Part 4 §5, §7: the compressor
 * and indexer frontiers are saved with the rows so a reload continues
 * mid-window; §6: state is written in logical order).  Layout, little-
 * endian: u32 magic 0x46345344 ("DS4F"), u32 version 1, u32 ratio, u32 coff,
 * u32 D_attn, u32 D_index (0 on ratio-128), u32 n_rot, u32 0; u64 n_tokens,
 * n_comp, n_index_comp; then float32 attention kv [coff*ratio, W_attn],
 * attention score, and on ratio-4 layers indexer kv and score.  Rows the
 * recurrence will overwrite before reading them are written as kv 0,
 * score -inf, so two runs that reach the same state write identical blobs.
 * Synchronises `stream`.  *written receives the blob size (may be NULL).
 * Errors: DS4C_EINVAL, DS4C_ECAP (cap too small), DS4C_EPOS, DS4C_EDEVICE. */
int ds4c_frontier_save(const ds4c_layer *layer, const ds4c_frontier *frontier,
                       void *host_buf, size_t cap, size_t *written, void *stream);

/* Restore a blob written by ds4c_frontier_save into an existing frontier
 * (Part 4 §12: restore copies bytes back into buffers that are already
 * allocated; nothing is mapped).  The header must match this layer exactly
 * (magic, version, ratio, coff, dims, n_rot), len must equal the blob size
 * and the counters must be consistent, else DS4C_EFORMAT and nothing
 * changes.  Synchronises `stream`. */
int ds4c_frontier_load(const ds4c_layer *layer, ds4c_frontier *frontier,
                       const void *host_buf, size_t len, void *stream);

/* A stack of layers (Part 3 §1: Flash layers 0-1 are uncompressed, then
 * ratio 4 and 128 alternate; §3: long prompts are prefilled in chunks of at
 * most 4096 tokens so windows stay on absolute positions).  Entry l of every
 * array belongs to layer l; a layer whose ratio is 0 has no compressor and
 * is skipped (its frontier and row entries are ignored and may be NULL).
 * Every layer reads the same x: the caller supplies each layer's input.
 *
 * ds4c_stack_workspace_bytes: workspace for chunks of up to chunk_cap tokens
 * (the largest need among the compressed layers).  0 if a descriptor is bad.
 *
 * ds4c_compress_stack_prefill: tokens x [T, hidden] at the frontiers'
 * positions, in chunks of chunk_cap (<= 0: ds4c_prefill_chunk_cap(T, 0));
 * for each chunk every layer in order.  All layers and the final row counts
 * are validated before anything is enqueued (same errors as
 * ds4c_compress_prefill; the frontiers must all be at the same position,
 * else DS4C_EPOS).  Asynchronous on `stream`.
 *
 * ds4c_compress_stack_decode_one: one token x [hidden] through every layer.
 *
 * ds4c_compress_stack_decode: n_tokens single-token decode steps, token
 * after token, each through every layer in order (Part 3 §4: the decode
 * path stores one token per call and pools at each window boundary); x is
 * [n_tokens, hidden], row t the input of step t.  Equivalent to n_tokens
 * calls of ds4c_compress_stack_decode_one, with the whole run validated
 * (positions, row capacity at the last step) before anything is enqueued.
 * Asynchronous on `stream`. */
size_t ds4c_stack_workspace_bytes(const ds4c_layer *layers, int n_layers, int64_t chunk_cap);
int ds4c_compress_stack_prefill(const ds4c_layer *layers, int n_layers, ds4c_frontier *frontiers,
                                const void *x, int64_t T, int64_t chunk_cap,
                                float *const *attn_rows, const int64_t *attn_cap,
                                float *const *index_rows, const int64_t *index_cap,
                                void *workspace, size_t ws_bytes, void *stream);
int ds4c_compress_stack_decode_one(const ds4c_layer *layers, int n_layers, ds4c_frontier *frontiers,
                                   const void *x, float *const *attn_rows, const int64_t *attn_cap,
                                   float *const *index_rows, const int64_t *index_cap, void *stream);
int ds4c_compress_stack_decode(const ds4c_layer *layers, int n_layers, ds4c_frontier *frontiers,
                               const void *x, int64_t n_tokens, float *const *attn_rows,
                               const int64_t *attn_cap, float *const *index_rows,
                               const int64_t *index_cap, void *stream);

/* Stack snapshot: the compressor's sections of a session payload (Part 4 §5:
 * per-layer compressed row counts, the compressed attention rows, the
 * compressor frontiers, the indexer rows and the indexer frontiers, in that
 * order; §6: rows 0 .. the live count, which are contiguous; §7: the
 * frontiers, so a reload continues mid-window).  The payload's other sections
 * (tokens, logits, raw sliding-window rows) belong to the caller.
 *
 * Layout, little-endian: u32 magic "DS4S" (0x53345344), u32 version 1,
 * u32 n_layers, u32 0, u64 n_tokens; per layer u32 ratio, D_attn, D_index,
 * n_rot (all 0 for an uncompressed layer); u32[n_layers] attention row
 * counts; u32[n_layers] indexer row counts; then float32 sections: each
 * compressed layer's rows [count, D_attn]; each compressed layer's attention
 * frontier kv then score [coff*ratio, W]; each ratio-4 layer's indexer rows
 * [count, D_index]; each ratio-4 layer's indexer frontier kv then score.
 * Frontier rows the recurrence never reads again are written as kv 0,
 * score -inf, so equal states give equal bytes.
 *
 * ds4c_stack_snapshot_bytes: the exact size for a stack at position n_tokens
 * (0 if a descriptor is invalid).
 * ds4c_stack_snapshot_save: every compressed layer's frontier must be at the
 * same position (else DS4C_EPOS); attn_rows[l] / index_rows[l] are the
 * layers' row buffers (device).  Copies to host_buf (host memory, cap bytes)
 * and synchronises the stream; *written receives the size.  DS4C_ECAP if cap
 * is too small.
 * ds4c_stack_snapshot_load: refuses (DS4C_EFORMAT) a buffer whose magic,
 * version, layer count, layer shapes, counts or length do not match; DS4C_ECAP
 * if a row buffer's capacity (rows) is too small.  Copies rows and frontier
 * tensors into the caller's existing device buffers (Part 4 §12), sets the
 * counters and synchronises the stream.  Nothing is written on a refusal. */
/* Indexer scoring and top-k of one query token over a ratio-4 layer's
 * compressed indexer rows (Part 3 §6: 64 heads of 128 dims, top 512 rows
 * reach the attention; Part 3 §9: the query passes the same Hadamard + FP4
 * round trip as the rows).  The score of row j is
 *   s_j = sum_h head_w[h] * max(0, <qhat_h, row_j>),
 * qhat_h = the round trip of q[h] (rotation by the orthonormal Hadamard
 * matrix of size head_dim, FP4 E2M1 in blocks of 32 with a power-of-two
 * scale; it stays rotated, like the rows).  The dot products run on bf16
 * matrix cores with float accumulation, each row value split into two bf16
 * parts: exact products for rows on the FP4 grid (as the compressor writes
 * them), and otherwise within 2^-16 of each float product.  The k rows
 * with the largest scores are written to out_idx / out_score (min(n_rows, k)
 * entries) in descending score order, equal scores to the lower row index.
 *
 * q [n_heads, head_dim], head_w [n_heads], index_rows [n_rows, head_dim]
 * (row-major float32, device; q and index_rows 16-byte aligned): the layer's
 * rows 0 .. n_index_comp-1 as ds4c_compress_* wrote them.  head_dim 64 or
 * 128; n_heads a multiple of 4 up to 64; 1 <= k <= 512; rows in chunks of
 * 32768 with ceil(n_rows / 32768) * k <= 16384 (n_rows up to 1,048,576 at
 * k = 512), else DS4C_ESHAPE.  q_hat (nullable, [n_heads, head_dim]) receives
 * the rotated, quantised query; scores (nullable, [n_rows]) every row's
 * score.  workspace: device, >= ds4c_indexer_workspace_bytes(n_rows, k),
 * 256-byte aligned.  Asynchronous on stream; n_rows == 0 writes nothing. */
size_t ds4c_indexer_workspace_bytes(int64_t n_rows, int32_t k);
int ds4c_indexer_topk(const float *q, const float *head_w, int32_t n_heads, int32_t head_dim,
                      const float *index_rows, int64_t n_rows, int32_t k, int32_t *out_idx, float *out_score,
                      float *q_hat, float *scores, void *workspace, size_t ws_bytes, void *stream);

/* ds4c_indexer_topk without a workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Same arguments, results and errors as
 * ds4c_indexer_topk; the scratch is a fixed array in the library, 8,519,936
 * bytes per device (every call of up to 1,048,576 rows fits), held by each
 * device the library runs on until the process ends.  Calls whose
 * ds4c_indexer_workspace_bytes(n_rows, k) exceeds it return DS4C_ECAP.  The
 * call allocates nothing (no hipMalloc, no events; kernel timing does not
 * cover it).  Every call on a device shares that device's array: calls that
 * overlap on one device (other streams, other threads) race and must be
 * serialised by the caller.  The stream must belong to the current device. */
int ds4c_indexer_topk_noalloc(const float *q, const float *head_w, int32_t n_heads, int32_t head_dim,
                              const float *index_rows, int64_t n_rows, int32_t k, int32_t *out_idx,
                              float *out_score, float *q_hat, float *scores, void *stream);

size_t ds4c_stack_snapshot_bytes(const ds4c_layer *layers, int n_layers, int64_t n_tokens);
int ds4c_stack_snapshot_save(const ds4c_layer *layers, int n_layers, const ds4c_frontier *frontiers,
                             const float *const *attn_rows, const float *const *index_rows, void *host_buf,
                             size_t cap, size_t *written, void *stream);
int ds4c_stack_snapshot_load(const ds4c_layer *layers, int n_layers, ds4c_frontier *frontiers,
                             float *const *attn_rows, const int64_t *attn_cap, float *const *index_rows,
                             const int64_t *index_cap, const void *host_buf, size_t len, void *stream);

/* Ratio-4 indexed mixed attention of one decode query (Part 3 §7).  The
 * query's n_heads heads attend, in one softmax, two sets of rows of
 * head_dim floats, each row serving as key and value for every head, with
 * logits <q_h, row> / sqrt(head_dim):
 *  - raw sliding-window rows: positions max(first_raw_pos, w0) ..
 *    min(qpos, raw_last_pos), where w0 = qpos + 1 - window when window > 0
 *    and qpos + 1 > window, else 0; position p is row p % ring_cap of
 *    raw_ring, which holds positions first_raw_pos .. raw_last_pos (none
 *    when raw_last_pos < first_raw_pos);
 *  - compressed rows: topk[0 .. k) walked in order, negative entries
 *    skipped, the walk ending at the first entry >= visible =
 *    (qpos + 1) / ratio (the rows the compressor has emitted by then); an
 *    entry listed twice is attended twice.
 * out[h] = sum_j softmax_j * row_j, or zeros when no row is attended.
 * Layout: q [n_heads, head_dim], raw_ring [ring_cap, head_dim], comp_rows
 * [n_comp, head_dim], out [n_heads, head_dim], all float32 row-major device
 * buffers, 16-byte aligned; topk int32 [k] (device).  n_heads a multiple of 8
 * in 8..128, head_dim 64/128/256/512 (else DS4C_ESHAPE, as for ring_cap or
 * k outside 0..4096); ratio >= 1, qpos >= 0, window >= 0, first_raw_pos >= 0
 * and at most ring_cap held positions (else DS4C_EINVAL); visible > n_comp
 * returns DS4C_ECAP.  The workspace (256-byte aligned, caller-owned,
 * ds4c_mixed_attention_workspace_bytes for the same n_heads, head_dim,
 * ring_cap and k) holds per-split partials.  Asynchronous on `stream`: two
 * launches, no allocation.  Timed as DS4C_KCLASS_ATTENTION. */
size_t ds4c_mixed_attention_workspace_bytes(int32_t n_heads, int32_t head_dim, int64_t ring_cap, int32_t k);
int ds4c_mixed_attention(const float *q, int32_t n_heads, int32_t head_dim, const float *raw_ring,
                         int64_t ring_cap, int64_t first_raw_pos, int64_t raw_last_pos, int64_t window,
                         const float *comp_rows, int64_t n_comp, const int32_t *topk, int32_t k, int64_t qpos,
                         int32_t ratio, float *out, void *workspace, size_t ws_bytes, void *stream);

/* Compress ratio of layer `layer` of a 0 = Flash / 1 = Pro model (Part 3
 * §1): Flash layers 0-1 -> 0 (uncompressed), Pro layers 0-1 -> 128; from
 * layer 2 even -> 4, odd -> 128.  -1 for a bad variant or negative layer. */
int ds4c_layer_ratio(int variant, int layer);

/* Prefill chunk cap (Part 3 §3): `override` if > 0, else 4096 when the
 * prompt is longer than 4096 tokens, else the prompt length (at least 1). */
int64_t ds4c_prefill_chunk_cap(int64_t prompt_len, int64_t override_cap);

/* Static description of a status code (Part 3 §1: the engine refuses to run
 * with a shape or layout it does not expect rather than guess; the codes name
 * which check refused a call); never NULL, also for codes the library does
 * not define. */
const char *ds4c_status_str(int status);

/* Kernel timing.  While enabled, every kernel of a selected class that the
 * library enqueues is bracketed by HIP events recorded by its own dispatch on
 * its stream; each bracket adds a few microseconds of queue time, so select
 * only the classes being measured.  class_mask: bit c selects class c
 * (DS4C_KCLASS_*), 0 turns timing off, DS4C_PROFILE_ALL selects every class;
 * other values return DS4C_EINVAL.  ds4c_profile_read waits for the recorded
 * events, writes the accumulated milliseconds and launch counts of each class
 * into ms[n] and count[n] (n <= DS4C_KCLASS_COUNT), and clears the record.
 * Enabling or disabling also clears it.  Classes: projection (PROJ; a
 * K-split call's plane sum included), pooling and row finishing (POOL), the
 * separate frontier-carry launch of a ratio-4 call that does not start on a
 * window boundary (CARRY), a decode step's projection (DECODE: the GEMV
 * launch) and its window-boundary pool (DECODE_POOL: the launches that pool,
 * finish and shift, only at a boundary), frontier init (INIT), indexer
 * scoring and top-k (INDEXER, the three launches of one call), mixed
 * attention (ATTENTION, the two launches of one call). */
enum { DS4C_KCLASS_PROJ = 0, DS4C_KCLASS_POOL = 1, DS4C_KCLASS_DECODE = 2, DS4C_KCLASS_INIT = 3,
       DS4C_KCLASS_CARRY = 4, DS4C_KCLASS_INDEXER = 5, DS4C_KCLASS_ATTENTION = 6,
       DS4C_KCLASS_DECODE_POOL = 7, DS4C_KCLASS_COUNT = 8 };
enum { DS4C_PROFILE_ALL = 0xFF };
int ds4c_profile_enable(int class_mask);
int ds4c_profile_read(double *ms, int64_t *count, int n);

/* Cold pool timings (measurement only).  While `scratch` is set and the
 * POOL class is being timed, every prefill call passes once over `bytes` of
 * `scratch` (a caller-owned device buffer, 16-byte aligned, bytes a multiple
 * of 16; 1 GiB exceeds the L2s and the 256 MiB Infinity Cache) between its
 * projection and its pooling launches, outside the timed interval, so the
 * pooling reads the projection output from HBM.  write = 0 reads the
 * buffer (the caches are left holding clean lines); write = 1 overwrites it
 * (the caches are left holding dirty lines, whose write-back then falls on
 * the pooling).  The buffer must stay allocated while set; its contents may
 * be overwritten in either mode.  (NULL, 0, 0) turns it off.  A NULL pointer
 * with nonzero bytes, a nonzero pointer with zero bytes, a misaligned
 * pointer or size, or write outside {0, 1} returns DS4C_EINVAL. */
int ds4c_profile_evict(void *scratch, size_t bytes, int write);

#ifdef __cplusplus
}
#endif

#endif /* DS4C_H */
