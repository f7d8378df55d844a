// Host-side checks of the C ABI's validation and blob parsing, built with
// AddressSanitizer and UndefinedBehaviorSanitizer around the library's host
// code (tests/test_abi_sanitize.py builds and runs it).  Every call here is
// refused before anything reaches the device, so no GPU is needed: the
// device pointers are aligned stand-ins that the library never dereferences
// on the host.  Blobs are heap copies of exactly the length passed, so a
// read past the end is an ASan report.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "ds4c.h"

namespace {

int g_fail = 0, g_checks = 0;

#define CHECK(c)                                                      \
  do {                                                                \
    ++g_checks;                                                       \
    if (!(c)) {                                                       \
      std::printf("FAIL %s:%d: %s\n", __FILE__, __LINE__, #c);        \
      ++g_fail;                                                       \
    }                                                                 \
  } while (0)

template <class T = void>
T* dev(uintptr_t a) {
  return reinterpret_cast<T*>(a);
}

ds4c_layer r4_layer() {
  ds4c_layer L{};
  L.ratio = 4;
  L.hidden = 256;
  L.n_rot = 64;
  L.in_dtype = DS4C_BF16;
  L.rope_base = 160000.f;
  L.rms_eps = 1e-6f;
  L.attn = {128, dev<const void>(0x100000), dev<const void>(0x200000), dev<const float>(0x300000),
            dev<const float>(0x400000)};
  L.index = {64, dev<const void>(0x500000), dev<const void>(0x600000), dev<const float>(0x700000),
             dev<const float>(0x800000)};
  return L;
}

ds4c_layer r128_layer() {
  ds4c_layer L = r4_layer();
  L.ratio = 128;
  L.attn.head_dim = 256;
  L.index = ds4c_lane{};
  return L;
}

void put_u32(std::vector<unsigned char>& b, size_t off, uint32_t v) { std::memcpy(b.data() + off, &v, 4); }
void put_u64(std::vector<unsigned char>& b, size_t off, uint64_t v) { std::memcpy(b.data() + off, &v, 8); }

void check_descriptors() {
  const ds4c_layer a = r4_layer(), b = r128_layer();
  CHECK(ds4c_frontier_bytes(&a) > 0);
  CHECK(ds4c_frontier_bytes(&b) > 0);
  CHECK(ds4c_frontier_bytes(nullptr) == 0);
  auto bad = [](ds4c_layer L) { return ds4c_frontier_bytes(&L) == 0; };
  ds4c_layer L = a;
  L.ratio = 0; CHECK(bad(L));
  L = a; L.ratio = 5; CHECK(bad(L));
  L = a; L.hidden = 100; CHECK(bad(L));
  L = a; L.hidden = 0; CHECK(bad(L));
  L = a; L.hidden = 16448; CHECK(bad(L));
  L = a; L.n_rot = 0; CHECK(bad(L));
  L = a; L.n_rot = 63; CHECK(bad(L));
  L = a; L.in_dtype = 7; CHECK(bad(L));
  L = a; L.rope_base = 0.f; CHECK(bad(L));
  L = a; L.rope_base = NAN; CHECK(bad(L));
  L = a; L.rms_eps = -1.f; CHECK(bad(L));
  L = a; L.attn.head_dim = 96; CHECK(bad(L));
  L = a; L.attn.head_dim = 1024; CHECK(bad(L));
  L = a; L.attn.wkv = nullptr; CHECK(bad(L));
  L = a; L.attn.wgate = dev<const void>(0x200004); CHECK(bad(L));
  L = a; L.index.head_dim = 0; CHECK(bad(L));
  L = a; L.index.ape = nullptr; CHECK(bad(L));
  L = b; L.index = a.index; CHECK(bad(L));
  CHECK(ds4c_workspace_bytes(&a, 4096) > 0);
  CHECK(ds4c_workspace_bytes(&a, -1) == 0);
  CHECK(ds4c_workspace_bytes(&a, int64_t(1) << 40) == 0);
  CHECK(ds4c_workspace_bytes(nullptr, 64) == 0);
  CHECK(ds4c_frontier_blob_bytes(&a) > 0);
  CHECK(ds4c_frontier_blob_bytes(nullptr) == 0);
}

void check_calls() {
  const ds4c_layer L = r4_layer();
  const size_t fb = ds4c_frontier_bytes(&L);
  (void)fb;
  ds4c_frontier f{0, 0, 0, dev(0x1000000)};
  void* x = dev(0x2000000);
  float* rows = dev<float>(0x3000000);
  float* irows = dev<float>(0x4000000);
  void* ws = dev(0x5000000);
  const size_t need = ds4c_workspace_bytes(&L, 4096);
  CHECK(ds4c_compress_prefill(nullptr, &f, x, 64, rows, 100, irows, 100, ws, need, nullptr, nullptr, nullptr) ==
        DS4C_EINVAL);
  CHECK(ds4c_compress_prefill(&L, nullptr, x, 64, rows, 100, irows, 100, ws, need, nullptr, nullptr, nullptr) ==
        DS4C_EINVAL);
  CHECK(ds4c_compress_prefill(&L, &f, nullptr, 64, rows, 100, irows, 100, ws, need, nullptr, nullptr, nullptr) !=
        DS4C_OK);
  CHECK(ds4c_compress_prefill(&L, &f, x, -1, rows, 100, irows, 100, ws, need, nullptr, nullptr, nullptr) != DS4C_OK);
  CHECK(ds4c_compress_prefill(&L, &f, x, 64, rows, 15, irows, 100, ws, need, nullptr, nullptr, nullptr) ==
        DS4C_ECAP);
  CHECK(ds4c_compress_prefill(&L, &f, x, 64, rows, 100, irows, 15, ws, need, nullptr, nullptr, nullptr) ==
        DS4C_ECAP);
  CHECK(ds4c_compress_prefill(&L, &f, x, 4096, rows, 2000, irows, 2000, ws, 256, nullptr, nullptr, nullptr) ==
        DS4C_ECAP);
  CHECK(ds4c_compress_prefill(&L, &f, dev(0x2000002), 64, rows, 100, irows, 100, ws, need, nullptr, nullptr,
                              nullptr) == DS4C_EINVAL);
  CHECK(ds4c_compress_prefill(&L, &f, x, 0, rows, 100, irows, 100, ws, need, nullptr, nullptr, nullptr) == DS4C_OK);
  ds4c_frontier g = f;
  g.n_tokens = 9;
  g.n_comp = 1;  // should be 2
  g.n_index_comp = 1;
  CHECK(ds4c_compress_prefill(&L, &g, x, 64, rows, 100, irows, 100, ws, need, nullptr, nullptr, nullptr) ==
        DS4C_EPOS);
  CHECK(ds4c_compress_decode_one(&L, &g, x, rows, 100, irows, 100, nullptr, nullptr, nullptr) == DS4C_EPOS);
  ds4c_frontier h{3, 0, 0, dev(0x1000000)};  // position 3: a window boundary
  CHECK(ds4c_compress_decode_one(&L, &h, x, rows, 0, irows, 100, nullptr, nullptr, nullptr) == DS4C_ECAP);
  CHECK(ds4c_compress_decode_one(&L, &h, nullptr, rows, 100, irows, 100, nullptr, nullptr, nullptr) != DS4C_OK);
  ds4c_frontier u{0, 0, 0, dev(0x1000010)};  // misaligned state
  CHECK(ds4c_compress_prefill(&L, &u, x, 64, rows, 100, irows, 100, ws, need, nullptr, nullptr, nullptr) ==
        DS4C_EINVAL);
  CHECK(f.n_tokens == 0 && f.n_comp == 0);  // refused calls change no counter
}

void check_frontier_blobs() {
  const ds4c_layer L = r4_layer();
  ds4c_frontier f{0, 0, 0, dev(0x1000000)};
  const size_t n = ds4c_frontier_blob_bytes(&L);
  std::vector<unsigned char> small(16);
  size_t written = 7;
  CHECK(ds4c_frontier_save(&L, &f, small.data(), small.size(), &written, nullptr) == DS4C_ECAP);
  // A well-formed header over a blob of the right size, then one field wrong
  // at a time; every variant is refused before any copy.
  std::vector<unsigned char> good(n, 0);
  put_u32(good, 0, 0x46345344u);
  put_u32(good, 4, 1);
  put_u32(good, 8, 4);
  put_u32(good, 12, 2);
  put_u32(good, 16, 128);
  put_u32(good, 20, 64);
  put_u32(good, 24, 64);
  put_u32(good, 28, 0);
  put_u64(good, 32, 9);
  put_u64(good, 40, 2);
  put_u64(good, 48, 2);
  struct Edit {
    size_t off;
    int width;
    uint64_t v;
  };
  const Edit edits[] = {{0, 4, 0x46345345u}, {4, 4, 2}, {8, 4, 128}, {12, 4, 1}, {16, 4, 256}, {20, 4, 0},
                        {24, 4, 32},         {28, 4, 1}, {40, 8, 3},  {48, 8, 0}, {32, 8, uint64_t(1) << 63}};
  for (const Edit& e : edits) {
    std::vector<unsigned char> b = good;
    if (e.width == 4) put_u32(b, e.off, uint32_t(e.v));
    else put_u64(b, e.off, e.v);
    CHECK(ds4c_frontier_load(&L, &f, b.data(), b.size(), nullptr) == DS4C_EFORMAT);
  }
  for (size_t len : {size_t(0), size_t(4), size_t(56), n - 1, n + 1}) {
    std::vector<unsigned char> b(good.begin(), good.begin() + std::min(len, n));
    b.resize(len);
    CHECK(ds4c_frontier_load(&L, &f, len ? b.data() : good.data(), len, nullptr) == DS4C_EFORMAT);
  }
  CHECK(ds4c_frontier_load(&L, &f, nullptr, n, nullptr) == DS4C_EINVAL);
  CHECK(f.n_tokens == 0);
}

void check_stack() {
  ds4c_layer layers[4] = {ds4c_layer{}, ds4c_layer{}, r4_layer(), r128_layer()};
  ds4c_frontier fr[4] = {{0, 0, 0, nullptr}, {0, 0, 0, nullptr}, {0, 0, 0, dev(0x1000000)},
                         {0, 0, 0, dev(0x1100000)}};
  CHECK(ds4c_stack_workspace_bytes(layers, 4, 4096) > 0);
  CHECK(ds4c_stack_workspace_bytes(layers, 4, 0) == 0);
  CHECK(ds4c_stack_workspace_bytes(nullptr, 4, 4096) == 0);
  CHECK(ds4c_stack_snapshot_bytes(layers, 4, 1000) > 0);
  CHECK(ds4c_stack_snapshot_bytes(layers, 4, -1) == 0);
  float* ar[4] = {nullptr, nullptr, dev<float>(0x3000000), dev<float>(0x3100000)};
  float* ir[4] = {nullptr, nullptr, dev<float>(0x4000000), nullptr};
  int64_t ac[4] = {0, 0, 1000, 100}, ic[4] = {0, 0, 1000, 0};
  // Frontiers at different positions.
  fr[3].n_tokens = 128;
  fr[3].n_comp = 1;
  CHECK(ds4c_compress_stack_prefill(layers, 4, fr, dev(0x2000000), 64, 0, ar, ac, ir, ic, dev(0x5000000),
                                    ds4c_stack_workspace_bytes(layers, 4, 4096), nullptr) == DS4C_EPOS);
  CHECK(ds4c_compress_stack_decode_one(layers, 4, fr, dev(0x2000000), ar, ac, ir, ic, nullptr) == DS4C_EPOS);
  CHECK(ds4c_compress_stack_decode(layers, 4, fr, dev(0x2000000), 16, ar, ac, ir, ic, nullptr) == DS4C_EPOS);
  fr[3].n_tokens = 0;
  fr[3].n_comp = 0;
  // 4004 decode steps from position 0 need 1001 ratio-4 rows; capacity is 1000.
  CHECK(ds4c_compress_stack_decode(layers, 4, fr, dev(0x2000000), 4004, ar, ac, ir, ic, nullptr) == DS4C_ECAP);
  CHECK(ds4c_compress_stack_decode(layers, 4, fr, dev(0x2000000), -1, ar, ac, ir, ic, nullptr) == DS4C_EINVAL);
  CHECK(ds4c_compress_stack_decode(layers, 4, fr, dev(0x2000000), 0, ar, ac, ir, ic, nullptr) == DS4C_OK);
  CHECK(ds4c_compress_stack_prefill(layers, 4, fr, dev(0x2000000), 64, 0, nullptr, ac, ir, ic, dev(0x5000000),
                                    ds4c_stack_workspace_bytes(layers, 4, 4096), nullptr) != DS4C_OK);
  // Snapshot headers: a consistent header for 1000 tokens over a blob that
  // is only the header long, then single-field corruptions and truncations.
  const size_t hdr = 24 + 24 * 4;
  std::vector<unsigned char> h(hdr, 0);
  put_u32(h, 0, 0x53345344u);
  put_u32(h, 4, 1);
  put_u32(h, 8, 4);
  put_u64(h, 16, 1000);
  const uint32_t desc[4][4] = {{0, 0, 0, 0}, {0, 0, 0, 0}, {4, 128, 64, 64}, {128, 256, 0, 64}};
  for (int l = 0; l < 4; ++l)
    for (int i = 0; i < 4; ++i) put_u32(h, 24 + 16 * l + 4 * i, desc[l][i]);
  const uint32_t cnt[4] = {0, 0, 250, 7}, icnt[4] = {0, 0, 250, 0};
  for (int l = 0; l < 4; ++l) {
    put_u32(h, 24 + 64 + 4 * l, cnt[l]);
    put_u32(h, 24 + 64 + 16 + 4 * l, icnt[l]);
  }
  CHECK(ds4c_stack_snapshot_load(layers, 4, fr, ar, ac, ir, ic, h.data(), h.size(), nullptr) == DS4C_EFORMAT);
  const size_t offs[] = {0, 4, 8, 12, 24 + 32, 24 + 36, 24 + 52, 24 + 64 + 8, 24 + 64 + 12, 24 + 80 + 8};
  for (size_t off : offs) {
    std::vector<unsigned char> b = h;
    put_u32(b, off, 12345);
    CHECK(ds4c_stack_snapshot_load(layers, 4, fr, ar, ac, ir, ic, b.data(), b.size(), nullptr) == DS4C_EFORMAT);
  }
  for (size_t len : {size_t(1), size_t(24), hdr - 1}) {
    std::vector<unsigned char> b(h.begin(), h.begin() + len);
    CHECK(ds4c_stack_snapshot_load(layers, 4, fr, ar, ac, ir, ic, b.data(), b.size(), nullptr) == DS4C_EFORMAT);
  }
  CHECK(ds4c_stack_snapshot_load(layers, 4, fr, ar, ac, ir, ic, nullptr, hdr, nullptr) == DS4C_EINVAL);
}

void check_next_rows_and_helpers() {
  const float* q = dev<const float>(0x100000);
  CHECK(ds4c_indexer_workspace_bytes(16448, 512) > 0);
  CHECK(ds4c_indexer_workspace_bytes(-1, 512) == 0);
  CHECK(ds4c_indexer_workspace_bytes(100, 513) == 0);
  CHECK(ds4c_indexer_workspace_bytes(int64_t(1) << 40, 512) == 0);
  int32_t* oi = dev<int32_t>(0x200000);
  float* os = dev<float>(0x300000);
  void* ws = dev(0x400000);
  CHECK(ds4c_indexer_topk(q, q, 64, 96, q, 100, 8, oi, os, nullptr, nullptr, ws, 1 << 20, nullptr) ==
        DS4C_ESHAPE);
  CHECK(ds4c_indexer_topk(q, q, 6, 128, q, 100, 8, oi, os, nullptr, nullptr, ws, 1 << 20, nullptr) == DS4C_ESHAPE);
  CHECK(ds4c_indexer_topk(q, q, 64, 128, q, 100, 0, oi, os, nullptr, nullptr, ws, 1 << 20, nullptr) ==
        DS4C_EINVAL);
  CHECK(ds4c_indexer_topk(q, q, 64, 128, q, 100, 8, oi, os, nullptr, nullptr, ws, 16, nullptr) == DS4C_ECAP);
  CHECK(ds4c_indexer_topk_noalloc(q, q, 64, 96, q, 100, 8, oi, os, nullptr, nullptr, nullptr) == DS4C_ESHAPE);
  CHECK(ds4c_indexer_topk_noalloc(q, q, 64, 128, q, 2000000, 1, oi, os, nullptr, nullptr, nullptr) == DS4C_ECAP);
  CHECK(ds4c_indexer_topk_noalloc(q, q, 64, 128, q, 0, 8, oi, os, nullptr, nullptr, nullptr) == DS4C_OK);
  CHECK(ds4c_mixed_attention_workspace_bytes(64, 512, 128, 512) > 0);
  CHECK(ds4c_mixed_attention_workspace_bytes(60, 512, 128, 512) == 0);
  const size_t mw = ds4c_mixed_attention_workspace_bytes(64, 512, 128, 512);
  float* out = dev<float>(0x500000);
  CHECK(ds4c_mixed_attention(q, 64, 512, q, 128, 0, 99, 128, q, 24, oi, 512, 99, 4, out, ws, mw, nullptr) ==
        DS4C_ECAP);
  CHECK(ds4c_mixed_attention(q, 64, 512, q, 128, 0, 128, 128, q, 25, oi, 512, 99, 4, out, ws, mw, nullptr) ==
        DS4C_EINVAL);
  CHECK(ds4c_mixed_attention(q, 64, 512, q, 128, 0, 99, 128, q, 25, oi, 512, 99, 0, out, ws, mw, nullptr) ==
        DS4C_EINVAL);
  CHECK(ds4c_mixed_attention(q, 64, 512, q, 128, 0, 99, 128, q, 25, oi, 512, 99, 4, out, ws, mw - 1, nullptr) ==
        DS4C_ECAP);
  for (int s = -20; s <= 20; ++s) CHECK(ds4c_status_str(s) != nullptr && ds4c_status_str(s)[0] != '\0');
  CHECK(ds4c_layer_ratio(0, 0) == 0 && ds4c_layer_ratio(0, 2) == 4 && ds4c_layer_ratio(0, 3) == 128);
  CHECK(ds4c_layer_ratio(1, 0) == 128 && ds4c_layer_ratio(2, 0) == -1 && ds4c_layer_ratio(0, -1) == -1);
  CHECK(ds4c_prefill_chunk_cap(10000, 0) == 4096 && ds4c_prefill_chunk_cap(100, 0) == 100);
  CHECK(ds4c_prefill_chunk_cap(0, 0) == 1 && ds4c_prefill_chunk_cap(10000, 512) == 512);
  CHECK(ds4c_profile_enable(-1) == DS4C_EINVAL && ds4c_profile_enable(DS4C_PROFILE_ALL + 1) == DS4C_EINVAL);
  double ms[DS4C_KCLASS_COUNT + 1];
  int64_t cnt[DS4C_KCLASS_COUNT + 1];
  CHECK(ds4c_profile_read(ms, cnt, DS4C_KCLASS_COUNT + 1) == DS4C_EINVAL);
  CHECK(ds4c_profile_read(nullptr, cnt, DS4C_KCLASS_COUNT) == DS4C_EINVAL);
  CHECK(ds4c_profile_read(ms, cnt, DS4C_KCLASS_COUNT) == DS4C_OK);
  CHECK(ds4c_profile_evict(nullptr, 16, 0) == DS4C_EINVAL && ds4c_profile_evict(dev(0x1008), 64, 0) == DS4C_EINVAL);
  CHECK(ds4c_profile_evict(dev(0x1000), 64, 3) == DS4C_EINVAL && ds4c_profile_evict(nullptr, 0, 0) == DS4C_OK);
}

}  // namespace

int main() {
  check_descriptors();
  check_calls();
  check_frontier_blobs();
  check_stack();
  check_next_rows_and_helpers();
  std::printf("%d checks, %d failed\n", g_checks, g_fail);
  if (g_fail == 0) std::printf("ALL OK\n");
  return g_fail ? 1 : 0;
}
