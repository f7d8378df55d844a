// C-ABI entry points of the compressor library: argument validation, launch
// plans, frontier counters, frontier save/load and optional kernel timing.
// Every check runs before anything is enqueued; nothing here touches the
// HIP runtime until the arguments have been accepted.
#include "ds4c.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <vector>

#include "kernel_args.h"
#include "launch.h"

namespace {

using ds4c::DecodeArgs;
using ds4c::FillArgs;
using ds4c::LaneDev;
using ds4c::PoolArgs;
using ds4c::ProjArgs;

constexpr size_t kCtrlBytes = 256;
constexpr int64_t kMaxTokensPerCall = int64_t(1) << 22;
constexpr int64_t kMaxRing = 4096;  // mixed attention: raw ring rows
constexpr int32_t kMaxTopk = 4096;  // mixed attention: list entries
constexpr uint32_t kBlobMagic = 0x46345344u;  // "DS4F" little-endian
constexpr uint32_t kBlobVersion = 1;
constexpr size_t kBlobHeader = 8 * 4 + 3 * 8;

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }
bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2_in(int v, int lo, int hi) { return v >= lo && v <= hi && (v & (v - 1)) == 0; }

struct Shape {
  int ratio = 0, coff = 0, n_lanes = 0;
  int D[2] = {0, 0}, W[2] = {0, 0};
  int N = 0;  // projection columns
  size_t fr_tensor_bytes[2] = {0, 0};
};

int check_lane(const ds4c_lane& l, const ds4c_layer& L, bool attn) {
  if (!pow2_in(l.head_dim, 64, 512)) return DS4C_ESHAPE;
  if (L.n_rot > l.head_dim) return DS4C_ESHAPE;
  if (attn && (l.head_dim - L.n_rot) % 64 != 0) return DS4C_ESHAPE;
  if (!l.wkv || !l.wgate || !l.ape || !l.norm_w) return DS4C_EINVAL;
  if (!aligned(l.wkv, 16) || !aligned(l.wgate, 16) || !aligned(l.ape, 16) || !aligned(l.norm_w, 16))
    return DS4C_EINVAL;
  return DS4C_OK;
}

int check_layer(const ds4c_layer* L, Shape* s) {
  if (!L) return DS4C_EINVAL;
  if (L->ratio != 4 && L->ratio != 128) return DS4C_EINVAL;
  if (L->in_dtype != DS4C_F32 && L->in_dtype != DS4C_BF16) return DS4C_EINVAL;
  if (!(std::isfinite(L->rope_base) && L->rope_base > 0.f)) return DS4C_EINVAL;
  if (!(std::isfinite(L->rms_eps) && L->rms_eps >= 0.f)) return DS4C_EINVAL;
  if (L->hidden <= 0 || L->hidden % 64 != 0 || L->hidden > 16384) return DS4C_ESHAPE;
  if (L->n_rot <= 0 || L->n_rot % 2 != 0) return DS4C_ESHAPE;
  int st = check_lane(L->attn, *L, true);
  if (st) return st;
  const ds4c_lane& ix = L->index;
  if (L->ratio == 4) {
    st = check_lane(ix, *L, false);
    if (st) return st;
  } else if (ix.head_dim != 0 || ix.wkv || ix.wgate || ix.ape || ix.norm_w) {
    return DS4C_EINVAL;
  }
  s->ratio = L->ratio;
  s->coff = L->ratio == 4 ? 2 : 1;
  s->n_lanes = L->ratio == 4 ? 2 : 1;
  s->N = 0;
  for (int l = 0; l < s->n_lanes; ++l) {
    s->D[l] = l == 0 ? L->attn.head_dim : ix.head_dim;
    s->W[l] = s->coff * s->D[l];
    s->N += 2 * s->W[l];
    s->fr_tensor_bytes[l] = size_t(s->coff) * L->ratio * s->W[l] * sizeof(float);
  }
  return DS4C_OK;
}

size_t frontier_bytes(const Shape& s) {
  size_t b = kCtrlBytes;
  for (int l = 0; l < s.n_lanes; ++l) b += 2 * s.fr_tensor_bytes[l];
  return b;
}

size_t blob_bytes(const Shape& s) { return kBlobHeader + frontier_bytes(s) - kCtrlBytes; }

// Device addresses of a lane's frontier tensors inside `state`.
void frontier_ptrs(const Shape& s, void* state, int lane, float** kv, float** sc) {
  char* p = static_cast<char*>(state) + kCtrlBytes;
  for (int l = 0; l < lane; ++l) p += 2 * s.fr_tensor_bytes[l];
  *kv = reinterpret_cast<float*>(p);
  *sc = reinterpret_cast<float*>(p + s.fr_tensor_bytes[lane]);
}

struct WsLayout {
  size_t proj = 0, part = 0, total = 0;
  int64_t max_rows = 0;
  // Fused ratio 4 (calls with n0 % 4 == 0), in the same buffer.
  size_t f_o = 0, f_part = 0, f_stage = 0;
};

// Plain path: projection [T, N] float32, then on ratio-128 layers the pool
// partials: per emitted row, 2 token halves x (max, sum, weighted sum) x D
// floats.  Fused ratio-4 path: pooled rows [T/4, D_attn + D_idx], the
// tile-start partials [ceil(T/256)][2][3][D_attn + D_idx] and the tokens
// the frontier keeps [7, N].  The buffer holds the larger of the two.
WsLayout workspace_layout(const Shape& s, int64_t T) {
  WsLayout w;
  w.proj = 0;
  // A K-split projection of a short call writes up to
  // max(T, min(kSplitRows, 16 T)) rows of partial sums.
  const int64_t split_rows = std::min(ds4c::kSplitRows, 16 * T);
  size_t off = align256(size_t(std::max(T, split_rows)) * s.N * sizeof(float));
  if (s.ratio == 128) {
    w.max_rows = T / 128 + 1;
    w.part = off;
    off += align256(size_t(w.max_rows) * 2 * 3 * s.D[0] * sizeof(float));
  }
  w.total = off;
  if (s.ratio == 4) {
    const size_t d_tot = size_t(s.D[0]) + size_t(s.n_lanes > 1 ? s.D[1] : 0);
    w.f_o = 0;
    size_t f = align256(size_t(T / 4 + 1) * d_tot * sizeof(float));
    w.f_part = f;
    f += align256(size_t((T + 255) / 256 + 1) * 2 * 3 * d_tot * sizeof(float));
    w.f_stage = f;
    f += align256(size_t(7) * s.N * sizeof(float));
    if (f > w.total) w.total = f;
  } else {
    // Fused ratio 128: pooled rows [T/128, D] and up to 127 kept tokens [127, N].
    w.f_o = 0;
    size_t f = align256(size_t(T / 128 + 1) * s.D[0] * sizeof(float));
    w.f_stage = f;
    f += align256(size_t(127) * s.N * sizeof(float));
    if (f > w.total) w.total = f;
  }
  return w;
}

int check_frontier(const Shape& s, const ds4c_frontier* f) {
  if (!f || !f->state || !aligned(f->state, 256)) return DS4C_EINVAL;
  if (f->n_tokens < 0) return DS4C_EPOS;
  if (f->n_comp != f->n_tokens / s.ratio) return DS4C_EPOS;
  if (f->n_index_comp != (s.ratio == 4 ? f->n_tokens / 4 : 0)) return DS4C_EPOS;
  return DS4C_OK;
}

int check_rows(const Shape& s, int64_t k_hi, int64_t n_emit, float* attn_rows, int64_t attn_cap,
               float* index_rows, int64_t index_cap, float* attn_pre, float* index_pre) {
  if (attn_cap < 0 || index_cap < 0) return DS4C_EINVAL;
  if (s.ratio == 128 && (index_rows || index_cap || index_pre)) return DS4C_EINVAL;
  if (!aligned(attn_rows, 16) || !aligned(index_rows, 16) || !aligned(attn_pre, 16) ||
      !aligned(index_pre, 16))
    return DS4C_EINVAL;
  if (n_emit > 0) {
    if (!attn_rows) return DS4C_EINVAL;
    if (k_hi > attn_cap) return DS4C_ECAP;
    if (s.ratio == 4) {
      if (!index_rows) return DS4C_EINVAL;
      if (k_hi > index_cap) return DS4C_ECAP;
    }
  }
  return DS4C_OK;
}

LaneDev lane_dev(const Shape& s, const ds4c_layer& L, void* state, int l, float* rows, float* pre) {
  const ds4c_lane& src = l == 0 ? L.attn : L.index;
  LaneDev d{};
  d.ape = src.ape;
  d.norm_w = src.norm_w;
  d.rows = rows;
  d.prequant = pre;
  frontier_ptrs(s, state, l, &d.fr_kv, &d.fr_sc);
  d.D = s.D[l];
  d.W = s.W[l];
  d.kv_col = l == 0 ? 0 : 2 * s.W[0];
  d.sc_col = d.kv_col + s.W[l];
  d.is_index = l;
  return d;
}

// ---------------------------------------------------------------------------
// Kernel timing with HIP events.
// ---------------------------------------------------------------------------
struct ProfRec {
  int cls;
  hipEvent_t a, b;
};
std::mutex g_prof_mu;
int g_prof_mask = 0;  // bit c: kernels of class c are timed
std::vector<ProfRec> g_prof;
std::vector<hipEvent_t> g_event_pool;
void* g_evict = nullptr;  // cold pool timings: buffer written before each timed pool
size_t g_evict_bytes = 0;
bool g_evict_write = false;

hipEvent_t take_event() {
  if (!g_event_pool.empty()) {
    hipEvent_t e = g_event_pool.back();
    g_event_pool.pop_back();
    return e;
  }
  // Timing-only events: without the system-scope fence a recorded event
  // does not write back and invalidate the caches, which would otherwise add
  // to the bracketed interval and slow the work that follows.
  hipEvent_t e = nullptr;
  if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
  return e;
}

void release_records() {
  for (auto& r : g_prof) {
    g_event_pool.push_back(r.a);
    g_event_pool.push_back(r.b);
  }
  g_prof.clear();
}

// Runs launch(Timing) and, while timing is on, records the interval of the
// kernels it enqueues under class `cls`.
template <class F>
hipError_t timed(int cls, F&& launch) {
  std::unique_lock<std::mutex> lk(g_prof_mu);
  if (!(g_prof_mask & (1 << cls))) {
    lk.unlock();
    return launch(ds4c::Timing{});
  }
  hipEvent_t a = take_event(), b = take_event();
  if (!a || !b) return hipErrorOutOfMemory;
  const hipError_t e = launch(ds4c::Timing{a, b});
  if (e != hipSuccess) return e;
  g_prof.push_back({cls, a, b});
  return hipSuccess;
}

// As timed(), for a launch sequence with two timed parts: the first under
// class `cls`, the second (present only when `has_second`) under `cls2`.
template <class F>
hipError_t timed2(int cls, int cls2, bool has_second, F&& launch) {
  std::unique_lock<std::mutex> lk(g_prof_mu);
  const bool on1 = g_prof_mask & (1 << cls), on2 = has_second && (g_prof_mask & (1 << cls2));
  if (!on1 && !on2) {
    lk.unlock();
    return launch(ds4c::Timing{}, ds4c::Timing{});
  }
  ds4c::Timing t1, t2;
  if (on1 && (!(t1.start = take_event()) || !(t1.stop = take_event()))) return hipErrorOutOfMemory;
  if (on2 && (!(t2.start = take_event()) || !(t2.stop = take_event()))) return hipErrorOutOfMemory;
  const hipError_t e = launch(t1, t2);
  if (e != hipSuccess) return e;
  if (on1) g_prof.push_back({cls, t1.start, t1.stop});
  if (on2) g_prof.push_back({cls2, t2.start, t2.stop});
  return hipSuccess;
}

int dev_status(hipError_t e) { return e == hipSuccess ? DS4C_OK : DS4C_EDEVICE; }

void fill_proj_segments(const ds4c_layer& L, const Shape& s, ds4c::ProjSeg* seg, int* n_seg) {
  int n = 0, col = 0;
  for (int l = 0; l < s.n_lanes; ++l) {
    const ds4c_lane& src = l == 0 ? L.attn : L.index;
    seg[n++] = {src.wkv, col, s.W[l]};
    col += s.W[l];
    seg[n++] = {src.wgate, col, s.W[l]};
    col += s.W[l];
  }
  *n_seg = n;
}

// Live frontier rows after n tokens (rows the recurrence will read again):
// ratio 4 keeps rows 0..3 once a window has been emitted and rows 4..3+c;
// ratio 128 keeps rows 0..c-1, with c = n % ratio.
bool row_live(int ratio, int64_t n, int row) {
  const int64_t c = n % ratio, m = n - c;
  if (ratio == 4) return row < 4 ? m >= 4 : row - 4 < c;
  return row < c;
}

void put_u32(unsigned char* p, uint32_t v) { std::memcpy(p, &v, 4); }
void put_u64(unsigned char* p, uint64_t v) { std::memcpy(p, &v, 8); }
uint32_t get_u32(const unsigned char* p) { uint32_t v; std::memcpy(&v, p, 4); return v; }
uint64_t get_u64(const unsigned char* p) { uint64_t v; std::memcpy(&v, p, 8); return v; }

// ---------------------------------------------------------------------------
// Stack snapshot: the compressor's sections of a session payload (Part 4 §5:
// per-layer compressed row counts, compressed attention rows, compressor
// frontiers, indexer rows, indexer frontiers, in that order; §6: rows 0 .. the
// live count are contiguous; §7: the frontiers make a reload continue
// mid-window).  Layout, little-endian:
//   u32 magic "DS4S", u32 version, u32 n_layers, u32 0, u64 n_tokens,
//   per layer u32 ratio, D_attn, D_idx, n_rot (0, 0, 0, 0 if uncompressed),
//   u32[n_layers] attention row counts, u32[n_layers] indexer row counts,
//   then per compressed layer its rows [count, D_attn] float32, then per
//   compressed layer its attention frontier kv and score, then per ratio-4
//   layer its indexer rows [count, D_idx], then per ratio-4 layer its indexer
//   frontier kv and score.  Frontier rows the recurrence never reads again
//   are written as kv 0, score -inf.
// ---------------------------------------------------------------------------
constexpr uint32_t kSnapMagic = 0x53345344u;  // "DS4S" little-endian
constexpr uint32_t kSnapVersion = 1;

size_t snap_header_bytes(int n_layers) { return 24 + 16 * size_t(n_layers) + 8 * size_t(n_layers); }

// Shapes of the stack's layers (ratio 0 -> uncompressed, shape.ratio = 0).
int snap_shapes(const ds4c_layer* layers, int n_layers, std::vector<Shape>* shapes) {
  if (!layers || n_layers <= 0) return DS4C_EINVAL;
  shapes->assign(size_t(n_layers), Shape{});
  for (int l = 0; l < n_layers; ++l) {
    if (layers[l].ratio == 0) continue;
    const int st = check_layer(&layers[l], &(*shapes)[size_t(l)]);
    if (st) return st;
  }
  return DS4C_OK;
}

size_t snap_bytes(const std::vector<Shape>& shapes, int64_t n) {
  size_t b = snap_header_bytes(int(shapes.size()));
  for (const Shape& s : shapes) {
    if (!s.ratio) continue;
    b += size_t(n / s.ratio) * size_t(s.D[0]) * 4 + 2 * s.fr_tensor_bytes[0];
    if (s.n_lanes > 1) b += size_t(n / 4) * size_t(s.D[1]) * 4 + 2 * s.fr_tensor_bytes[1];
  }
  return b;
}

// Byte offsets of the four body sections' entries of layer l (rows, frontier).
struct SnapOffsets {
  std::vector<size_t> attn_rows, attn_fr, idx_rows, idx_fr;
};

SnapOffsets snap_offsets(const std::vector<Shape>& shapes, int64_t n) {
  SnapOffsets o;
  const size_t L = shapes.size();
  o.attn_rows.assign(L, 0);
  o.attn_fr.assign(L, 0);
  o.idx_rows.assign(L, 0);
  o.idx_fr.assign(L, 0);
  size_t off = snap_header_bytes(int(L));
  for (size_t l = 0; l < L; ++l)
    if (shapes[l].ratio) { o.attn_rows[l] = off; off += size_t(n / shapes[l].ratio) * size_t(shapes[l].D[0]) * 4; }
  for (size_t l = 0; l < L; ++l)
    if (shapes[l].ratio) { o.attn_fr[l] = off; off += 2 * shapes[l].fr_tensor_bytes[0]; }
  for (size_t l = 0; l < L; ++l)
    if (shapes[l].n_lanes > 1) { o.idx_rows[l] = off; off += size_t(n / 4) * size_t(shapes[l].D[1]) * 4; }
  for (size_t l = 0; l < L; ++l)
    if (shapes[l].n_lanes > 1) { o.idx_fr[l] = off; off += 2 * shapes[l].fr_tensor_bytes[1]; }
  return o;
}

// Position shared by every compressed layer's frontier, or -1.
int64_t snap_position(const std::vector<Shape>& shapes, const ds4c_frontier* frontiers) {
  int64_t n = -1;
  for (size_t l = 0; l < shapes.size(); ++l) {
    if (!shapes[l].ratio) continue;
    if (check_frontier(shapes[l], &frontiers[l])) return -1;
    if (n >= 0 && frontiers[l].n_tokens != n) return -1;
    n = frontiers[l].n_tokens;
  }
  return n < 0 ? 0 : n;
}

}  // namespace

extern "C" {

size_t ds4c_frontier_bytes(const ds4c_layer* layer) {
  Shape s;
  return check_layer(layer, &s) ? 0 : frontier_bytes(s);
}

size_t ds4c_workspace_bytes(const ds4c_layer* layer, int64_t max_tokens) {
  Shape s;
  if (check_layer(layer, &s) || max_tokens < 0 || max_tokens > kMaxTokensPerCall) return 0;
  return workspace_layout(s, max_tokens).total;
}

size_t ds4c_frontier_blob_bytes(const ds4c_layer* layer) {
  Shape s;
  return check_layer(layer, &s) ? 0 : blob_bytes(s);
}

int ds4c_frontier_init(const ds4c_layer* layer, ds4c_frontier* frontier, void* stream) {
  try {
    Shape s;
    int st = check_layer(layer, &s);
    if (st) return st;
    if (!frontier || !frontier->state || !aligned(frontier->state, 256)) return DS4C_EINVAL;
    FillArgs f{};
    f.n_lanes = s.n_lanes;
    for (int l = 0; l < s.n_lanes; ++l) {
      frontier_ptrs(s, frontier->state, l, &f.kv[l], &f.sc[l]);
      f.n[l] = int64_t(s.fr_tensor_bytes[l] / sizeof(float));
    }
    f.ctrl = static_cast<unsigned*>(frontier->state);
    f.n_ctrl = int(kCtrlBytes / sizeof(unsigned));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    st = dev_status(timed(DS4C_KCLASS_INIT, [&](const ds4c::Timing& tm) { return ds4c::launch_fill(f, hs, tm); }));
    if (st) return st;
    frontier->n_tokens = frontier->n_comp = frontier->n_index_comp = 0;
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_compress_prefill(const ds4c_layer* layer, ds4c_frontier* frontier, const void* x, int64_t T,
                          float* attn_rows, int64_t attn_cap, float* index_rows, int64_t index_cap,
                          void* workspace, size_t ws_bytes, float* attn_prequant, float* index_prequant,
                          void* stream) {
  try {
    Shape s;
    int st = check_layer(layer, &s);
    if (st) return st;
    st = check_frontier(s, frontier);
    if (st) return st;
    if (T < 0) return DS4C_EINVAL;
    if (T > kMaxTokensPerCall) return DS4C_ESHAPE;
    const int r = s.ratio;
    const int64_t n0 = frontier->n_tokens, n = n0 + T;
    const int64_t k_lo = n0 / r, k_hi = n / r, n_emit = k_hi - k_lo;
    st = check_rows(s, k_hi, n_emit, attn_rows, attn_cap, index_rows, index_cap, attn_prequant,
                    index_prequant);
    if (st) return st;
    if (T == 0) return DS4C_OK;
    if (!x || !aligned(x, 16)) return DS4C_EINVAL;
    const WsLayout wl = workspace_layout(s, T);
    if (!workspace || !aligned(workspace, 256)) return DS4C_EINVAL;
    if (ws_bytes < wl.total) return DS4C_ECAP;
    // One token is one step of the recurrence: the decode path does it in
    // one GEMV launch (plus the pool launch at a window boundary) instead of
    // a projection, a plane sum, a pool and a carry launch.
    if (T == 1)
      return ds4c_compress_decode_one(layer, frontier, x, attn_rows, attn_cap, index_rows, index_cap, attn_prequant,
                                      index_prequant, stream);

    char* ws = static_cast<char*>(workspace);
    ProjArgs pa{};
    pa.x = x;
    pa.out = reinterpret_cast<float*>(ws + wl.proj);
    pa.M = T;
    pa.K = layer->hidden;
    pa.N = s.N;
    fill_proj_segments(*layer, s, pa.seg, &pa.n_seg);
    // Window pooling joins the projection epilogue when the call starts on a
    // window boundary and the fused grid is wide enough; otherwise the plain
    // projection runs, with K split for short calls.
    const bool fused = n0 % r == 0 && ds4c::use_fused_projection(r, T, s.N, layer->hidden,
                                                                  s.D[0] + (s.n_lanes > 1 ? s.D[1] : 0));
    pa.k_split = fused ? 1 : ds4c::proj_plan(T, s.N, layer->hidden).k_split;
    pa.k_len = layer->hidden / pa.k_split;
    pa.split_stride = T * s.N;

    PoolArgs po{};
    po.proj = pa.out;
    po.ld = s.N;
    po.n0 = n0;
    po.T = T;
    po.k_lo = k_lo;
    po.k_hi = k_hi;
    po.ratio = r;
    po.n_rot = layer->n_rot;
    po.n_lanes = s.n_lanes;
    po.log2_base = std::log2((double)layer->rope_base);
    po.rms_eps = layer->rms_eps;
    po.lane[0] = lane_dev(s, *layer, frontier->state, 0, attn_rows, attn_prequant);
    if (s.n_lanes > 1) po.lane[1] = lane_dev(s, *layer, frontier->state, 1, index_rows, index_prequant);
    if (r == 128) po.part = reinterpret_cast<float*>(ws + wl.part);

    if (r == 128 && fused) {
      // Window pool fused into the projection epilogue (one 128-token tile
      // is one window); the pool launch finishes rows and carries the frontier.
      ds4c::FuseArgs& f = pa.fuse;
      f.on = 1;
      f.ratio = 128;
      f.d_attn = s.D[0];
      f.d_tot = s.D[0];
      f.W[0] = s.W[0];
      f.n_orig = s.N;
      f.n_emit = n_emit;
      f.carry_lo = T - T % 128;
      f.ape[0] = layer->attn.ape;
      f.o = reinterpret_cast<float*>(ws + wl.f_o);
      f.stage = reinterpret_cast<float*>(ws + wl.f_stage);
      po.o = f.o;
      po.stage = f.stage;
      po.d_tot = f.d_tot;
      po.carry_lo = f.carry_lo;
    }
    if (r == 4 && fused) {
      // Window pool fused into the projection epilogue; the pool launch
      // only finishes the rows and carries the frontier.
      const int64_t m_rel = T - T % 4;
      ds4c::FuseArgs& f = pa.fuse;
      f.on = 1;
      f.ratio = 4;
      f.d_attn = s.D[0];
      f.d_idx = s.n_lanes > 1 ? s.D[1] : 0;
      f.d_tot = f.d_attn + f.d_idx;
      f.W[0] = s.W[0];
      f.W[1] = s.n_lanes > 1 ? s.W[1] : 0;
      f.n_orig = s.N;
      f.n_emit = n_emit;
      f.carry_lo = m_rel >= 4 ? m_rel - 4 : 0;
      f.ape[0] = layer->attn.ape;
      f.ape[1] = s.n_lanes > 1 ? layer->index.ape : nullptr;
      f.o = reinterpret_cast<float*>(ws + wl.f_o);
      f.part = reinterpret_cast<float*>(ws + wl.f_part);
      f.stage = reinterpret_cast<float*>(ws + wl.f_stage);
      for (int l = 0; l < s.n_lanes; ++l) {
        float* kv = nullptr;
        float* sc = nullptr;
        frontier_ptrs(s, frontier->state, l, &kv, &sc);
        f.fr_kv[l] = kv;
        f.fr_sc[l] = sc;
      }
      po.o = f.o;
      po.part = f.part;
      po.stage = f.stage;
      po.d_tot = f.d_tot;
      po.carry_lo = f.carry_lo;
    }

    hipStream_t hs = static_cast<hipStream_t>(stream);
    st = dev_status(
        timed(DS4C_KCLASS_PROJ, [&](const ds4c::Timing& tm) { return ds4c::launch_proj(pa, layer->in_dtype, hs, tm); }));
    if (st) return st;
    // The plain ratio-4 path's second launch only carries the frontier; it
    // is timed as its own class.
    const int n_pool = ds4c::pool_launches(po);
    const int n_main = r == 4 && !po.o ? n_pool - 1 : n_pool;
    {
      // Cold pool timings: evict the projection output from the caches
      // between the two launches, outside the timed interval.
      std::lock_guard<std::mutex> lk(g_prof_mu);
      if (g_evict && (g_prof_mask & (1 << DS4C_KCLASS_POOL)))
        st = dev_status(ds4c::launch_evict(g_evict, g_evict_bytes, g_evict_write, hs));
    }
    if (st) return st;
    st = dev_status(timed(DS4C_KCLASS_POOL, [&](const ds4c::Timing& tm) {
      hipError_t e = hipSuccess;
      for (int ph = 0; ph < n_main && e == hipSuccess; ++ph)
        e = ds4c::launch_pool(po, ph, hs,
                              ds4c::Timing{ph == 0 ? tm.start : nullptr, ph == n_main - 1 ? tm.stop : nullptr});
      return e;
    }));
    if (st) return st;
    if (n_main < n_pool) {
      st = dev_status(
          timed(DS4C_KCLASS_CARRY, [&](const ds4c::Timing& tm) { return ds4c::launch_pool(po, n_main, hs, tm); }));
      if (st) return st;
    }
    frontier->n_tokens = n;
    frontier->n_comp = k_hi;
    frontier->n_index_comp = r == 4 ? k_hi : 0;
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

namespace {

// Arguments of one decode step of a validated layer; the caller sets d.x and
// d.pos per token (everything else stays fixed for a layer).
DecodeArgs decode_args(const Shape& s, const ds4c_layer& layer, void* state, float* attn_rows, float* index_rows,
                       float* attn_prequant, float* index_prequant) {
  DecodeArgs d{};
  d.K = layer.hidden;
  d.N = s.N;
  fill_proj_segments(layer, s, d.seg, &d.n_seg);
  d.ratio = s.ratio;
  d.n_rot = layer.n_rot;
  d.n_lanes = s.n_lanes;
  d.log2_base = std::log2((double)layer.rope_base);
  d.rms_eps = layer.rms_eps;
  d.lane[0] = lane_dev(s, layer, state, 0, attn_rows, attn_prequant);
  if (s.n_lanes > 1) d.lane[1] = lane_dev(s, layer, state, 1, index_rows, index_prequant);
  return d;
}

// Enqueues the step at d.pos and advances the frontier's counters.
int enqueue_decode(const DecodeArgs& d, int in_dtype, ds4c_frontier* frontier, hipStream_t hs) {
  const int r = d.ratio;
  const int64_t pos = d.pos, k_hi = (pos + 1) / r;
  const bool boundary = (pos + 1) % r == 0;
  const int st = dev_status(timed2(DS4C_KCLASS_DECODE, DS4C_KCLASS_DECODE_POOL, boundary,
                                   [&](const ds4c::Timing& tm, const ds4c::Timing& tp) {
                                     return ds4c::launch_decode(d, in_dtype, hs, tm, tp);
                                   }));
  if (st) return st;
  frontier->n_tokens = pos + 1;
  frontier->n_comp = k_hi;
  frontier->n_index_comp = r == 4 ? k_hi : 0;
  return DS4C_OK;
}

}  // namespace

int ds4c_compress_decode_one(const ds4c_layer* layer, ds4c_frontier* frontier, const void* x,
                             float* attn_rows, int64_t attn_cap, float* index_rows, int64_t index_cap,
                             float* attn_prequant, float* index_prequant, void* stream) {
  try {
    Shape s;
    int st = check_layer(layer, &s);
    if (st) return st;
    st = check_frontier(s, frontier);
    if (st) return st;
    const int r = s.ratio;
    const int64_t pos = frontier->n_tokens;
    const int64_t k_hi = (pos + 1) / r, n_emit = k_hi - pos / r;
    st = check_rows(s, k_hi, n_emit, attn_rows, attn_cap, index_rows, index_cap, attn_prequant,
                    index_prequant);
    if (st) return st;
    if (!x || !aligned(x, 16)) return DS4C_EINVAL;
    DecodeArgs d = decode_args(s, *layer, frontier->state, attn_rows, index_rows, attn_prequant, index_prequant);
    d.x = x;
    d.pos = pos;
    return enqueue_decode(d, layer->in_dtype, frontier, static_cast<hipStream_t>(stream));
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_frontier_save(const ds4c_layer* layer, const ds4c_frontier* frontier, void* host_buf,
                       size_t cap, size_t* written, void* stream) {
  try {
    Shape s;
    int st = check_layer(layer, &s);
    if (st) return st;
    st = check_frontier(s, frontier);
    if (st) return st;
    if (!host_buf) return DS4C_EINVAL;
    const size_t need = blob_bytes(s);
    if (cap < need) return DS4C_ECAP;
    unsigned char* out = static_cast<unsigned char*>(host_buf);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    size_t off = kBlobHeader;
    for (int l = 0; l < s.n_lanes; ++l) {
      float *kv, *sc;
      frontier_ptrs(s, frontier->state, l, &kv, &sc);
      if (hipMemcpyAsync(out + off, kv, s.fr_tensor_bytes[l], hipMemcpyDeviceToHost, hs) != hipSuccess)
        return DS4C_EDEVICE;
      off += s.fr_tensor_bytes[l];
      if (hipMemcpyAsync(out + off, sc, s.fr_tensor_bytes[l], hipMemcpyDeviceToHost, hs) != hipSuccess)
        return DS4C_EDEVICE;
      off += s.fr_tensor_bytes[l];
    }
    if (hipStreamSynchronize(hs) != hipSuccess) return DS4C_EDEVICE;
    // Canonical form of rows the recurrence never reads again.
    off = kBlobHeader;
    const int rows = s.coff * s.ratio;
    for (int l = 0; l < s.n_lanes; ++l) {
      float* kv = reinterpret_cast<float*>(out + off);
      float* sc = reinterpret_cast<float*>(out + off + s.fr_tensor_bytes[l]);
      for (int row = 0; row < rows; ++row) {
        if (row_live(s.ratio, frontier->n_tokens, row)) continue;
        for (int c = 0; c < s.W[l]; ++c) {
          kv[size_t(row) * s.W[l] + c] = 0.f;
          sc[size_t(row) * s.W[l] + c] = -INFINITY;
        }
      }
      off += 2 * s.fr_tensor_bytes[l];
    }
    put_u32(out + 0, kBlobMagic);
    put_u32(out + 4, kBlobVersion);
    put_u32(out + 8, uint32_t(s.ratio));
    put_u32(out + 12, uint32_t(s.coff));
    put_u32(out + 16, uint32_t(s.D[0]));
    put_u32(out + 20, uint32_t(s.n_lanes > 1 ? s.D[1] : 0));
    put_u32(out + 24, uint32_t(layer->n_rot));
    put_u32(out + 28, 0u);
    put_u64(out + 32, uint64_t(frontier->n_tokens));
    put_u64(out + 40, uint64_t(frontier->n_comp));
    put_u64(out + 48, uint64_t(frontier->n_index_comp));
    if (written) *written = need;
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_frontier_load(const ds4c_layer* layer, ds4c_frontier* frontier, const void* host_buf, size_t len,
                       void* stream) {
  try {
    Shape s;
    int st = check_layer(layer, &s);
    if (st) return st;
    if (!frontier || !frontier->state || !aligned(frontier->state, 256) || !host_buf) return DS4C_EINVAL;
    const unsigned char* in = static_cast<const unsigned char*>(host_buf);
    if (len != blob_bytes(s)) return DS4C_EFORMAT;
    if (get_u32(in + 0) != kBlobMagic || get_u32(in + 4) != kBlobVersion) return DS4C_EFORMAT;
    if (get_u32(in + 8) != uint32_t(s.ratio) || get_u32(in + 12) != uint32_t(s.coff) ||
        get_u32(in + 16) != uint32_t(s.D[0]) ||
        get_u32(in + 20) != uint32_t(s.n_lanes > 1 ? s.D[1] : 0) ||
        get_u32(in + 24) != uint32_t(layer->n_rot) || get_u32(in + 28) != 0u)
      return DS4C_EFORMAT;
    const uint64_t nt = get_u64(in + 32), nc = get_u64(in + 40), ni = get_u64(in + 48);
    if (nt > uint64_t(INT64_MAX) || nc != nt / uint64_t(s.ratio) || ni != (s.ratio == 4 ? nt / 4 : 0))
      return DS4C_EFORMAT;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    size_t off = kBlobHeader;
    for (int l = 0; l < s.n_lanes; ++l) {
      float *kv, *sc;
      frontier_ptrs(s, frontier->state, l, &kv, &sc);
      if (hipMemcpyAsync(kv, in + off, s.fr_tensor_bytes[l], hipMemcpyHostToDevice, hs) != hipSuccess)
        return DS4C_EDEVICE;
      off += s.fr_tensor_bytes[l];
      if (hipMemcpyAsync(sc, in + off, s.fr_tensor_bytes[l], hipMemcpyHostToDevice, hs) != hipSuccess)
        return DS4C_EDEVICE;
      off += s.fr_tensor_bytes[l];
    }
    if (hipStreamSynchronize(hs) != hipSuccess) return DS4C_EDEVICE;
    frontier->n_tokens = int64_t(nt);
    frontier->n_comp = int64_t(nc);
    frontier->n_index_comp = int64_t(ni);
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

size_t ds4c_stack_workspace_bytes(const ds4c_layer* layers, int n_layers, int64_t chunk_cap) {
  if (!layers || n_layers <= 0 || chunk_cap <= 0 || chunk_cap > kMaxTokensPerCall) return 0;
  size_t need = 0;
  for (int l = 0; l < n_layers; ++l) {
    if (layers[l].ratio == 0) continue;
    Shape s;
    if (check_layer(&layers[l], &s)) return 0;
    const size_t b = workspace_layout(s, chunk_cap).total;
    need = b > need ? b : need;
  }
  return need;
}

int ds4c_compress_stack_prefill(const ds4c_layer* layers, int n_layers, ds4c_frontier* frontiers, const void* x,
                                int64_t T, int64_t chunk_cap, float* const* attn_rows, const int64_t* attn_cap,
                                float* const* index_rows, const int64_t* index_cap, void* workspace,
                                size_t ws_bytes, void* stream) {
  try {
    if (!layers || !frontiers || n_layers <= 0 || !attn_rows || !attn_cap || !index_rows || !index_cap)
      return DS4C_EINVAL;
    if (T < 0) return DS4C_EINVAL;
    if (chunk_cap <= 0) chunk_cap = ds4c_prefill_chunk_cap(T, 0);
    if (chunk_cap > kMaxTokensPerCall) return DS4C_ESHAPE;
    // Validate every compressed layer for the whole run before enqueueing.
    int64_t n0 = -1;
    int n_comp_layers = 0;
    for (int l = 0; l < n_layers; ++l) {
      if (layers[l].ratio == 0) continue;
      Shape s;
      int st = check_layer(&layers[l], &s);
      if (st) return st;
      st = check_frontier(s, &frontiers[l]);
      if (st) return st;
      if (n0 < 0) n0 = frontiers[l].n_tokens;
      if (frontiers[l].n_tokens != n0) return DS4C_EPOS;
      const int64_t k_lo = n0 / s.ratio, k_hi = (n0 + T) / s.ratio;
      st = check_rows(s, k_hi, k_hi - k_lo, attn_rows[l], attn_cap[l], index_rows[l], index_cap[l], nullptr,
                      nullptr);
      if (st) return st;
      ++n_comp_layers;
    }
    if (n_comp_layers == 0 || T == 0) return DS4C_OK;
    if (!x || !aligned(x, 16)) return DS4C_EINVAL;
    const int64_t chunk = chunk_cap < T ? chunk_cap : T;
    if (!workspace || !aligned(workspace, 256)) return DS4C_EINVAL;
    if (ws_bytes < ds4c_stack_workspace_bytes(layers, n_layers, chunk)) return DS4C_ECAP;
    // All layers read the same x: its row size is the first compressed layer's.
    size_t row_bytes = 0;
    for (int l = 0; l < n_layers; ++l) {
      if (layers[l].ratio == 0) continue;
      const size_t b = size_t(layers[l].hidden) * (layers[l].in_dtype == DS4C_BF16 ? 2 : 4);
      if (row_bytes == 0) row_bytes = b;
      if (b != row_bytes) return DS4C_ESHAPE;
    }
    for (int64_t t0 = 0; t0 < T; t0 += chunk) {
      const int64_t tc = T - t0 < chunk ? T - t0 : chunk;
      const void* xc = static_cast<const char*>(x) + size_t(t0) * row_bytes;
      for (int l = 0; l < n_layers; ++l) {
        if (layers[l].ratio == 0) continue;
        const int st = ds4c_compress_prefill(&layers[l], &frontiers[l], xc, tc, attn_rows[l], attn_cap[l],
                                             index_rows[l], index_cap[l], workspace, ws_bytes, nullptr, nullptr,
                                             stream);
        if (st) return st;  // only a HIP failure can get here
      }
    }
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_compress_stack_decode(const ds4c_layer* layers, int n_layers, ds4c_frontier* frontiers, const void* x,
                               int64_t n_tokens, float* const* attn_rows, const int64_t* attn_cap,
                               float* const* index_rows, const int64_t* index_cap, void* stream) {
  try {
    if (!layers || !frontiers || n_layers <= 0 || !attn_rows || !attn_cap || !index_rows || !index_cap)
      return DS4C_EINVAL;
    if (n_tokens < 0 || n_tokens > kMaxTokensPerCall) return DS4C_EINVAL;
    int64_t n0 = -1;
    size_t row_bytes = 0;
    for (int l = 0; l < n_layers; ++l) {
      if (layers[l].ratio == 0) continue;
      Shape s;
      int st = check_layer(&layers[l], &s);
      if (st) return st;
      st = check_frontier(s, &frontiers[l]);
      if (st) return st;
      if (n0 < 0) n0 = frontiers[l].n_tokens;
      if (frontiers[l].n_tokens != n0) return DS4C_EPOS;
      const int64_t k_hi = (n0 + n_tokens) / s.ratio;
      st = check_rows(s, k_hi, k_hi - n0 / s.ratio, attn_rows[l], attn_cap[l], index_rows[l], index_cap[l],
                      nullptr, nullptr);
      if (st) return st;
      // All layers read the same x rows: one row size for the stack.
      const size_t b = size_t(layers[l].hidden) * (layers[l].in_dtype == DS4C_BF16 ? 2 : 4);
      if (row_bytes == 0) row_bytes = b;
      if (b != row_bytes) return DS4C_ESHAPE;
    }
    if (n0 < 0 || n_tokens == 0) return DS4C_OK;
    if (!x || !aligned(x, 16)) return DS4C_EINVAL;
    // Everything is validated: build each layer's arguments once, then
    // enqueue token after token, each through every layer in order.
    std::vector<DecodeArgs> args(n_layers);
    for (int l = 0; l < n_layers; ++l) {
      if (layers[l].ratio == 0) continue;
      Shape s;
      check_layer(&layers[l], &s);
      args[l] = decode_args(s, layers[l], frontiers[l].state, attn_rows[l], index_rows[l], nullptr, nullptr);
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    for (int64_t t = 0; t < n_tokens; ++t) {
      const void* xt = static_cast<const char*>(x) + size_t(t) * row_bytes;
      for (int l = 0; l < n_layers; ++l) {
        if (layers[l].ratio == 0) continue;
        args[l].x = xt;
        args[l].pos = n0 + t;
        const int st = enqueue_decode(args[l], layers[l].in_dtype, &frontiers[l], hs);
        if (st) return st;  // only a HIP failure can get here
      }
    }
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_compress_stack_decode_one(const ds4c_layer* layers, int n_layers, ds4c_frontier* frontiers,
                                   const void* x, float* const* attn_rows, const int64_t* attn_cap,
                                   float* const* index_rows, const int64_t* index_cap, void* stream) {
  return ds4c_compress_stack_decode(layers, n_layers, frontiers, x, 1, attn_rows, attn_cap, index_rows, index_cap,
                                    stream);
}

int ds4c_layer_ratio(int variant, int layer) {
  if ((variant != 0 && variant != 1) || layer < 0) return -1;
  if (layer < 2) return variant == 0 ? 0 : 128;
  return layer % 2 == 0 ? 4 : 128;
}

int64_t ds4c_prefill_chunk_cap(int64_t prompt_len, int64_t override_cap) {
  if (override_cap > 0) return override_cap;
  if (prompt_len > 4096) return 4096;
  return prompt_len > 1 ? prompt_len : 1;
}

const char* ds4c_status_str(int status) {
  switch (status) {
    case DS4C_OK: return "ok";
    case DS4C_EINVAL: return "invalid argument";
    case DS4C_ESHAPE: return "unsupported shape";
    case DS4C_ECAP: return "buffer too small";
    case DS4C_EPOS: return "inconsistent frontier counters";
    case DS4C_EFORMAT: return "bad frontier blob";
    case DS4C_EDEVICE: return "HIP runtime error";
    default: return "unknown status";
  }
}

size_t ds4c_stack_snapshot_bytes(const ds4c_layer* layers, int n_layers, int64_t n_tokens) {
  try {
    std::vector<Shape> shapes;
    if (snap_shapes(layers, n_layers, &shapes) || n_tokens < 0 || n_tokens > (int64_t(1) << 40)) return 0;
    return snap_bytes(shapes, n_tokens);
  } catch (...) {
    return 0;
  }
}

int ds4c_stack_snapshot_save(const ds4c_layer* layers, int n_layers, const ds4c_frontier* frontiers,
                             const float* const* attn_rows, const float* const* index_rows, void* host_buf,
                             size_t cap, size_t* written, void* stream) {
  try {
    std::vector<Shape> shapes;
    int st = snap_shapes(layers, n_layers, &shapes);
    if (st) return st;
    if (!frontiers || !attn_rows || !index_rows || !host_buf) return DS4C_EINVAL;
    const int64_t n = snap_position(shapes, frontiers);
    if (n < 0) return DS4C_EPOS;
    for (int l = 0; l < n_layers; ++l) {
      const Shape& sh = shapes[size_t(l)];
      if (!sh.ratio) continue;
      if (n / sh.ratio > 0 && !attn_rows[l]) return DS4C_EINVAL;
      if (sh.n_lanes > 1 && n / 4 > 0 && !index_rows[l]) return DS4C_EINVAL;
      if (n / sh.ratio > int64_t(UINT32_MAX)) return DS4C_ESHAPE;
    }
    const size_t need = snap_bytes(shapes, n);
    if (cap < need) return DS4C_ECAP;
    unsigned char* out = static_cast<unsigned char*>(host_buf);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const SnapOffsets o = snap_offsets(shapes, n);
    for (int l = 0; l < n_layers; ++l) {
      const Shape& sh = shapes[size_t(l)];
      if (!sh.ratio) continue;
      for (int ln = 0; ln < sh.n_lanes; ++ln) {
        const int64_t cnt = n / (ln ? 4 : sh.ratio);
        const float* rows = ln ? index_rows[l] : attn_rows[l];
        unsigned char* dst_rows = out + (ln ? o.idx_rows[size_t(l)] : o.attn_rows[size_t(l)]);
        if (cnt > 0 && hipMemcpyAsync(dst_rows, rows, size_t(cnt) * size_t(sh.D[ln]) * 4, hipMemcpyDeviceToHost,
                                      hs) != hipSuccess)
          return DS4C_EDEVICE;
        float *kv, *sc;
        frontier_ptrs(sh, frontiers[l].state, ln, &kv, &sc);
        unsigned char* dst_fr = out + (ln ? o.idx_fr[size_t(l)] : o.attn_fr[size_t(l)]);
        if (hipMemcpyAsync(dst_fr, kv, sh.fr_tensor_bytes[ln], hipMemcpyDeviceToHost, hs) != hipSuccess ||
            hipMemcpyAsync(dst_fr + sh.fr_tensor_bytes[ln], sc, sh.fr_tensor_bytes[ln], hipMemcpyDeviceToHost, hs) !=
                hipSuccess)
          return DS4C_EDEVICE;
      }
    }
    if (hipStreamSynchronize(hs) != hipSuccess) return DS4C_EDEVICE;
    // Header and counts; canonical form of frontier rows never read again.
    put_u32(out + 0, kSnapMagic);
    put_u32(out + 4, kSnapVersion);
    put_u32(out + 8, uint32_t(n_layers));
    put_u32(out + 12, 0u);
    put_u64(out + 16, uint64_t(n));
    for (int l = 0; l < n_layers; ++l) {
      const Shape& sh = shapes[size_t(l)];
      unsigned char* d = out + 24 + 16 * size_t(l);
      put_u32(d + 0, uint32_t(sh.ratio));
      put_u32(d + 4, uint32_t(sh.ratio ? sh.D[0] : 0));
      put_u32(d + 8, uint32_t(sh.n_lanes > 1 ? sh.D[1] : 0));
      put_u32(d + 12, uint32_t(sh.ratio ? layers[l].n_rot : 0));
      unsigned char* c = out + 24 + 16 * size_t(n_layers) + 4 * size_t(l);
      put_u32(c, uint32_t(sh.ratio ? n / sh.ratio : 0));
      put_u32(c + 4 * size_t(n_layers), uint32_t(sh.n_lanes > 1 ? n / 4 : 0));
      for (int ln = 0; ln < sh.n_lanes; ++ln) {
        float* kv = reinterpret_cast<float*>(out + (ln ? o.idx_fr[size_t(l)] : o.attn_fr[size_t(l)]));
        float* sc = kv + sh.fr_tensor_bytes[ln] / 4;
        for (int row = 0; row < sh.coff * sh.ratio; ++row) {
          if (row_live(sh.ratio, n, row)) continue;
          for (int cc = 0; cc < sh.W[ln]; ++cc) {
            kv[size_t(row) * sh.W[ln] + cc] = 0.f;
            sc[size_t(row) * sh.W[ln] + cc] = -INFINITY;
          }
        }
      }
    }
    if (written) *written = need;
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_stack_snapshot_load(const ds4c_layer* layers, int n_layers, ds4c_frontier* frontiers,
                             float* const* attn_rows, const int64_t* attn_cap, float* const* index_rows,
                             const int64_t* index_cap, const void* host_buf, size_t len, void* stream) {
  try {
    std::vector<Shape> shapes;
    int st = snap_shapes(layers, n_layers, &shapes);
    if (st) return st;
    if (!frontiers || !attn_rows || !attn_cap || !index_rows || !index_cap || !host_buf) return DS4C_EINVAL;
    const unsigned char* in = static_cast<const unsigned char*>(host_buf);
    if (len < snap_header_bytes(n_layers)) return DS4C_EFORMAT;
    if (get_u32(in + 0) != kSnapMagic || get_u32(in + 4) != kSnapVersion ||
        get_u32(in + 8) != uint32_t(n_layers) || get_u32(in + 12) != 0u)
      return DS4C_EFORMAT;
    const uint64_t nt = get_u64(in + 16);
    if (nt > (uint64_t(1) << 40)) return DS4C_EFORMAT;
    const int64_t n = int64_t(nt);
    for (int l = 0; l < n_layers; ++l) {
      const Shape& sh = shapes[size_t(l)];
      const unsigned char* d = in + 24 + 16 * size_t(l);
      const unsigned char* c = in + 24 + 16 * size_t(n_layers) + 4 * size_t(l);
      if (get_u32(d) != uint32_t(sh.ratio) || get_u32(d + 4) != uint32_t(sh.ratio ? sh.D[0] : 0) ||
          get_u32(d + 8) != uint32_t(sh.n_lanes > 1 ? sh.D[1] : 0) ||
          get_u32(d + 12) != uint32_t(sh.ratio ? layers[l].n_rot : 0))
        return DS4C_EFORMAT;
      if (get_u32(c) != uint32_t(sh.ratio ? n / sh.ratio : 0) ||
          get_u32(c + 4 * size_t(n_layers)) != uint32_t(sh.n_lanes > 1 ? n / 4 : 0))
        return DS4C_EFORMAT;
    }
    if (len != snap_bytes(shapes, n)) return DS4C_EFORMAT;
    for (int l = 0; l < n_layers; ++l) {
      const Shape& sh = shapes[size_t(l)];
      if (!sh.ratio) continue;
      if (!frontiers[l].state || !aligned(frontiers[l].state, 256)) return DS4C_EINVAL;
      if (attn_cap[l] < n / sh.ratio || (n / sh.ratio > 0 && !attn_rows[l])) return DS4C_ECAP;
      if (sh.n_lanes > 1 && (index_cap[l] < n / 4 || (n / 4 > 0 && !index_rows[l]))) return DS4C_ECAP;
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const SnapOffsets o = snap_offsets(shapes, n);
    for (int l = 0; l < n_layers; ++l) {
      const Shape& sh = shapes[size_t(l)];
      if (!sh.ratio) continue;
      for (int ln = 0; ln < sh.n_lanes; ++ln) {
        const int64_t cnt = n / (ln ? 4 : sh.ratio);
        float* rows = ln ? index_rows[l] : attn_rows[l];
        const unsigned char* src_rows = in + (ln ? o.idx_rows[size_t(l)] : o.attn_rows[size_t(l)]);
        if (cnt > 0 && hipMemcpyAsync(rows, src_rows, size_t(cnt) * size_t(sh.D[ln]) * 4, hipMemcpyHostToDevice,
                                      hs) != hipSuccess)
          return DS4C_EDEVICE;
        float *kv, *sc;
        frontier_ptrs(sh, frontiers[l].state, ln, &kv, &sc);
        const unsigned char* src_fr = in + (ln ? o.idx_fr[size_t(l)] : o.attn_fr[size_t(l)]);
        if (hipMemcpyAsync(kv, src_fr, sh.fr_tensor_bytes[ln], hipMemcpyHostToDevice, hs) != hipSuccess ||
            hipMemcpyAsync(sc, src_fr + sh.fr_tensor_bytes[ln], sh.fr_tensor_bytes[ln], hipMemcpyHostToDevice, hs) !=
                hipSuccess)
          return DS4C_EDEVICE;
      }
    }
    if (hipStreamSynchronize(hs) != hipSuccess) return DS4C_EDEVICE;
    for (int l = 0; l < n_layers; ++l) {
      const Shape& sh = shapes[size_t(l)];
      if (!sh.ratio) continue;
      frontiers[l].n_tokens = n;
      frontiers[l].n_comp = n / sh.ratio;
      frontiers[l].n_index_comp = sh.ratio == 4 ? n / 4 : 0;
    }
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

size_t ds4c_indexer_workspace_bytes(int64_t n_rows, int32_t k) {
  if (n_rows < 0 || k < 1 || k > 512) return 0;
  const int64_t chunks = (n_rows + ds4c::kIndexerChunk - 1) / ds4c::kIndexerChunk;
  if (chunks * k > ds4c::kIndexerMaxCand) return 0;
  const size_t hist_words = size_t((n_rows + 63) / 64) * 64;  // 64 words of first-digit counts per 64-row block
  return align256(size_t(n_rows) * 4) + align256(size_t(chunks) * size_t(k) * 8) + align256(hist_words * 4) + 256;
}

namespace {

// Validates an indexer call (everything but the workspace) and fills its
// arguments; the scores default to the workspace's first section.
int indexer_args(const float* q, const float* head_w, int32_t n_heads, int32_t head_dim, const float* index_rows,
                 int64_t n_rows, int32_t k, int32_t* out_idx, float* out_score, float* q_hat, float* scores,
                 size_t* need, ds4c::IndexerArgs* a) {
  if (head_dim != 64 && head_dim != 128) return DS4C_ESHAPE;
  if (n_heads < 4 || n_heads > 64 || n_heads % 4 != 0) return DS4C_ESHAPE;
  if (k < 1 || k > 512 || n_rows < 0) return DS4C_EINVAL;
  *need = ds4c_indexer_workspace_bytes(n_rows, k);
  if (*need == 0) return DS4C_ESHAPE;
  if (!q || !head_w || !aligned(q, 16) || !aligned(head_w, 4)) return DS4C_EINVAL;
  if (n_rows > 0 && (!index_rows || !aligned(index_rows, 16))) return DS4C_EINVAL;
  if (!out_idx || !out_score) return DS4C_EINVAL;
  if (q_hat && !aligned(q_hat, 16)) return DS4C_EINVAL;
  *a = ds4c::IndexerArgs{};
  a->q = q;
  a->head_w = head_w;
  a->rows = index_rows;
  a->n = n_rows;
  a->H = n_heads;
  a->Dh = head_dim;
  a->scores = scores;
  a->q_hat = q_hat;
  a->out_idx = out_idx;
  a->out_score = out_score;
  a->k = k;
  a->n_chunks = int((n_rows + ds4c::kIndexerChunk - 1) / ds4c::kIndexerChunk);
  return DS4C_OK;
}

void indexer_workspace(ds4c::IndexerArgs* a, char* ws) {
  if (!a->scores) a->scores = reinterpret_cast<float*>(ws);
  const size_t cand_off = align256(size_t(a->n) * 4);
  a->cand = reinterpret_cast<uint64_t*>(ws + cand_off);
  a->hist = reinterpret_cast<uint32_t*>(ws + cand_off + align256(size_t(a->n_chunks) * size_t(a->k) * 8));
}

}  // namespace

int ds4c_indexer_topk(const float* q, const float* head_w, int32_t n_heads, int32_t head_dim,
                      const float* index_rows, int64_t n_rows, int32_t k, int32_t* out_idx, float* out_score,
                      float* q_hat, float* scores, void* workspace, size_t ws_bytes, void* stream) {
  try {
    size_t need = 0;
    ds4c::IndexerArgs a;
    const int st = indexer_args(q, head_w, n_heads, head_dim, index_rows, n_rows, k, out_idx, out_score, q_hat,
                                scores, &need, &a);
    if (st) return st;
    if (!workspace || !aligned(workspace, 256)) return DS4C_EINVAL;
    if (ws_bytes < need) return DS4C_ECAP;
    if (n_rows == 0) return DS4C_OK;
    indexer_workspace(&a, static_cast<char*>(workspace));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return dev_status(
        timed(DS4C_KCLASS_INDEXER, [&](const ds4c::Timing& tm) { return ds4c::launch_indexer(a, hs, tm); }));
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_indexer_topk_noalloc(const float* q, const float* head_w, int32_t n_heads, int32_t head_dim,
                              const float* index_rows, int64_t n_rows, int32_t k, int32_t* out_idx,
                              float* out_score, float* q_hat, float* scores, void* stream) {
  try {
    size_t need = 0;
    ds4c::IndexerArgs a;
    const int st = indexer_args(q, head_w, n_heads, head_dim, index_rows, n_rows, k, out_idx, out_score, q_hat,
                                scores, &need, &a);
    if (st) return st;
    if (need > ds4c::kIndexerScratchBytes) return DS4C_ECAP;
    if (n_rows == 0) return DS4C_OK;
    void* ws = nullptr;
    if (ds4c::indexer_scratch(&ws) != hipSuccess) return DS4C_EDEVICE;
    indexer_workspace(&a, static_cast<char*>(ws));
    // Untimed: the timing mode may create events, which this entry point must not.
    return dev_status(ds4c::launch_indexer(a, static_cast<hipStream_t>(stream), ds4c::Timing{}));
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

size_t ds4c_mixed_attention_workspace_bytes(int32_t n_heads, int32_t head_dim, int64_t ring_cap, int32_t k) {
  if (n_heads < 8 || n_heads > 128 || n_heads % 8 != 0) return 0;
  if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512) return 0;
  if (ring_cap < 0 || ring_cap > kMaxRing || k < 0 || k > kMaxTopk) return 0;
  const size_t splits = size_t(ds4c::mixed_attn_splits(int(ring_cap + k)));
  return align256(splits * n_heads * head_dim * 4) + 2 * align256(splits * n_heads * 4);
}

int ds4c_mixed_attention(const float* q, int32_t n_heads, int32_t head_dim, const float* raw_ring, int64_t ring_cap,
                         int64_t first_raw_pos, int64_t raw_last_pos, int64_t window, const float* comp_rows,
                         int64_t n_comp, const int32_t* topk, int32_t k, int64_t qpos, int32_t ratio, float* out,
                         void* workspace, size_t ws_bytes, void* stream) {
  try {
    const size_t need = ds4c_mixed_attention_workspace_bytes(n_heads, head_dim, ring_cap, k);
    if (need == 0) return DS4C_ESHAPE;
    if (ratio < 1 || qpos < 0 || window < 0 || n_comp < 0 || first_raw_pos < 0) return DS4C_EINVAL;
    if (!q || !aligned(q, 16) || !out || !aligned(out, 16)) return DS4C_EINVAL;
    // The ring holds positions first_raw_pos .. raw_last_pos (none when
    // raw_last_pos < first_raw_pos), at most ring_cap of them.
    if (raw_last_pos >= first_raw_pos && raw_last_pos - first_raw_pos + 1 > ring_cap) return DS4C_EINVAL;
    const int64_t window_first = (window != 0 && qpos + 1 > window) ? qpos + 1 - window : 0;
    const int64_t first = std::max(first_raw_pos, window_first), last = std::min(qpos, raw_last_pos);
    const int64_t n_raw = last >= first ? last - first + 1 : 0;
    if (n_raw > 0 && (!raw_ring || !aligned(raw_ring, 16))) return DS4C_EINVAL;
    const int64_t visible = (qpos + 1) / ratio;
    if (visible > n_comp) return DS4C_ECAP;
    if (visible > 0 && (!comp_rows || !aligned(comp_rows, 16))) return DS4C_EINVAL;
    if (k > 0 && (!topk || !aligned(topk, 4))) return DS4C_EINVAL;
    if (!workspace || !aligned(workspace, 256)) return DS4C_EINVAL;
    if (ws_bytes < need) return DS4C_ECAP;
    char* ws = static_cast<char*>(workspace);
    ds4c::MixedAttnArgs a{};
    a.q = q;
    a.ring = raw_ring;
    a.comp = comp_rows;
    a.topk = topk;
    a.H = n_heads;
    a.D = head_dim;
    a.ring_cap = int(ring_cap);
    a.ring_row0 = ring_cap > 0 ? int(first % ring_cap) : 0;
    a.k = k;
    a.n_raw = int(n_raw);
    a.visible = visible;
    a.n_split = ds4c::mixed_attn_splits(int(n_raw + k));
    a.scale = float(1.0 / std::sqrt(double(head_dim)));
    const size_t o_bytes = align256(size_t(a.n_split) * n_heads * head_dim * 4);
    const size_t ml_bytes = align256(size_t(a.n_split) * n_heads * 4);
    a.part_o = reinterpret_cast<float*>(ws);
    a.part_m = reinterpret_cast<float*>(ws + o_bytes);
    a.part_l = reinterpret_cast<float*>(ws + o_bytes + ml_bytes);
    a.out = out;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    return dev_status(timed(DS4C_KCLASS_ATTENTION,
                            [&](const ds4c::Timing& tm) { return ds4c::launch_mixed_attention(a, hs, tm); }));
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_profile_enable(int class_mask) {
  try {
    if (class_mask < 0 || class_mask > DS4C_PROFILE_ALL) return DS4C_EINVAL;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    release_records();
    g_prof_mask = class_mask;
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_profile_evict(void* scratch, size_t bytes, int write) {
  try {
    if ((scratch == nullptr) != (bytes == 0) || (write != 0 && write != 1)) return DS4C_EINVAL;
    if (reinterpret_cast<uintptr_t>(scratch) % 16 || bytes % 16) return DS4C_EINVAL;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    g_evict = scratch;
    g_evict_bytes = bytes;
    g_evict_write = write == 1;
    return DS4C_OK;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

int ds4c_profile_read(double* ms, int64_t* count, int n) {
  try {
    if (!ms || !count || n < 0 || n > DS4C_KCLASS_COUNT) return DS4C_EINVAL;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    for (int i = 0; i < n; ++i) {
      ms[i] = 0.0;
      count[i] = 0;
    }
    int st = DS4C_OK;
    for (auto& r : g_prof) {
      if (hipEventSynchronize(r.b) != hipSuccess) {
        st = DS4C_EDEVICE;
        continue;
      }
      float t = 0.f;
      if (hipEventElapsedTime(&t, r.a, r.b) != hipSuccess) {
        st = DS4C_EDEVICE;
        continue;
      }
      if (r.cls < n) {
        ms[r.cls] += t;
        count[r.cls] += 1;
      }
    }
    release_records();
    return st;
  } catch (...) {
    return DS4C_EDEVICE;
  }
}

}  // extern "C"
