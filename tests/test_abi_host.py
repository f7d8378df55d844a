"""The C-ABI library on the host, without a GPU.

The library must load and export every symbol include/ds4c.h declares.  Every
call here fails validation (or is host-only), so nothing is enqueued: the
error paths must return their exact status before touching the HIP runtime.
"""

import ctypes
import os
import re
import struct

import numpy as np
import pytest

import oracle
from compressed_kv_attention_compressor_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds4c.h")

FAKE = 0x7F0000000000  # 256-byte aligned, never dereferenced


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ds4c_[a-z0-9_]+)\s*\(", text)))


def make_layer(ratio=4, hidden=4096, da=512, di=128, dtype=B.DS4C_BF16, n_rot=64):
    L = B.Layer()
    L.ratio, L.hidden, L.n_rot, L.in_dtype = ratio, hidden, n_rot, dtype
    L.rope_base, L.rms_eps = 160000.0, 1e-6
    L.attn = B.Lane(da, FAKE, FAKE + 0x100000, FAKE + 0x200000, FAKE + 0x300000)
    if ratio == 4:
        L.index = B.Lane(di, FAKE + 0x400000, FAKE + 0x500000, FAKE + 0x600000, FAKE + 0x700000)
    return L


def frontier(n=0, ratio=4):
    f = B.Frontier()
    f.n_tokens, f.n_comp, f.n_index_comp = n, n // ratio, (n // 4 if ratio == 4 else 0)
    f.state = FAKE + 0x10000000
    return f


def test_library_exports_every_declared_symbol():
    lib = B.lib()
    names = declared_functions()
    assert len(names) == 26
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(B.SIGNATURES), "binding and header disagree"


def test_sizes():
    L = make_layer()
    assert B.ds4c_frontier_bytes(L) == 256 + 2 * 8 * 1024 * 4 + 2 * 8 * 256 * 4
    assert B.ds4c_workspace_bytes(L, 4096) == 4096 * 2560 * 4
    assert B.ds4c_frontier_blob_bytes(L) == 56 + 2 * 8 * 1024 * 4 + 2 * 8 * 256 * 4
    L3 = make_layer(ratio=128)
    assert B.ds4c_frontier_bytes(L3) == 256 + 2 * 128 * 512 * 4
    # projection + pool partials [33 rows, 2 halves, 3, 512], 256-aligned
    ws = 4096 * 1024 * 4 + ((33 * 2 * 3 * 512 * 4 + 255) // 256) * 256
    assert B.ds4c_workspace_bytes(L3, 4096) == ws
    assert B.ds4c_frontier_bytes(make_layer(ratio=3)) == 0


def test_schedule_helpers_match_oracle():
    for layer in range(40):
        assert B.ds4c_layer_ratio(0, layer) == oracle.layer_compress_ratio(layer, "flash")
        assert B.ds4c_layer_ratio(1, layer) == oracle.layer_compress_ratio(layer, "pro")
    assert B.ds4c_layer_ratio(2, 5) == -1
    for n in (1, 100, 4096, 4097, 65536):
        assert B.ds4c_prefill_chunk_cap(n, 0) == oracle.prefill_chunk_cap(n)
    assert B.ds4c_prefill_chunk_cap(65536, 512) == 512


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -5, -6, -99):
        assert isinstance(B.status_str(code), str) and B.status_str(code)


def _prefill(L, f, T=64, attn_cap=10**6, index_cap=10**6, ws=None, x=FAKE + 0x20000000, index_rows=None):
    ws_bytes = B.ds4c_workspace_bytes(L, T) if ws is None else ws
    idx = (FAKE + 0x40000000 if L.ratio == 4 else 0) if index_rows is None else index_rows
    return B.lib().ds4c_compress_prefill(ctypes.byref(L), ctypes.byref(f), x, T,
                                         FAKE + 0x30000000, attn_cap, idx, index_cap if L.ratio == 4 else 0,
                                         FAKE + 0x50000000, ws_bytes, 0, 0, None)


@pytest.mark.parametrize("mutate,status", [
    (lambda L, f: setattr(L, "ratio", 0), B.DS4C_EINVAL),
    (lambda L, f: setattr(L, "ratio", 8), B.DS4C_EINVAL),
    (lambda L, f: setattr(L, "in_dtype", 7), B.DS4C_EINVAL),
    (lambda L, f: setattr(L, "rope_base", -1.0), B.DS4C_EINVAL),
    (lambda L, f: setattr(L, "rms_eps", float("nan")), B.DS4C_EINVAL),
    (lambda L, f: setattr(L, "hidden", 100), B.DS4C_ESHAPE),
    (lambda L, f: setattr(L, "n_rot", 63), B.DS4C_ESHAPE),
    (lambda L, f: setattr(L.attn, "head_dim", 384), B.DS4C_ESHAPE),
    (lambda L, f: setattr(L.attn, "head_dim", 1024), B.DS4C_ESHAPE),
    (lambda L, f: setattr(L, "n_rot", 32), B.DS4C_ESHAPE),  # 512 - 32 not a whole FP8 block
    (lambda L, f: setattr(L.index, "head_dim", 96), B.DS4C_ESHAPE),
    (lambda L, f: setattr(L.attn, "wkv", None), B.DS4C_EINVAL),
    (lambda L, f: setattr(L.index, "norm_w", FAKE + 4), B.DS4C_EINVAL),
    (lambda L, f: setattr(f, "state", None), B.DS4C_EINVAL),
    (lambda L, f: setattr(f, "state", FAKE + 16), B.DS4C_EINVAL),
    (lambda L, f: setattr(f, "n_comp", 3), B.DS4C_EPOS),
    (lambda L, f: setattr(f, "n_tokens", -4), B.DS4C_EPOS),
])
def test_prefill_rejects_bad_arguments(mutate, status):
    L, f = make_layer(), frontier(n=8)
    mutate(L, f)
    before = (f.n_tokens, f.n_comp, f.n_index_comp)
    assert _prefill(L, f) == status
    assert (f.n_tokens, f.n_comp, f.n_index_comp) == before


def test_prefill_capacity_and_workspace():
    L = make_layer()
    f = frontier(n=8)  # rows 0, 1 already appended; 64 more tokens -> rows up to 17
    assert _prefill(L, f, T=64, attn_cap=17) == B.DS4C_ECAP
    assert _prefill(L, f, T=64, index_cap=17) == B.DS4C_ECAP
    assert _prefill(L, f, T=64, ws=B.ds4c_workspace_bytes(L, 64) - 1) == B.DS4C_ECAP
    assert _prefill(L, f, T=-1) == B.DS4C_EINVAL
    assert _prefill(L, f, T=64, x=FAKE + 8) == B.DS4C_EINVAL
    assert _prefill(L, f, T=1 << 23) == B.DS4C_ESHAPE
    # a ratio-128 layer must not be given indexer rows
    L3, f3 = make_layer(ratio=128), frontier(ratio=128)
    assert B.lib().ds4c_compress_prefill(ctypes.byref(L3), ctypes.byref(f3), FAKE, 64, FAKE, 10, FAKE, 10,
                                         FAKE, 1 << 30, 0, 0, None) == B.DS4C_EINVAL
    # ratio 128 with an indexer lane is refused
    L3.index = B.Lane(128, FAKE, FAKE, FAKE, FAKE)
    assert _prefill(L3, f3) == B.DS4C_EINVAL
    # ratio 4 with no indexer lane is refused
    L4 = make_layer()
    L4.index = B.Lane()
    assert _prefill(L4, frontier()) == B.DS4C_ESHAPE


def test_prefill_zero_tokens_is_a_noop():
    L, f = make_layer(), frontier(n=5)
    assert _prefill(L, f, T=0) == B.DS4C_OK
    assert (f.n_tokens, f.n_comp) == (5, 1)


def test_decode_rejects_bad_arguments():
    L, f = make_layer(), frontier(n=7)  # position 7 closes window 1 -> needs cap >= 2
    lib = B.lib()
    args = lambda cap: (ctypes.byref(L), ctypes.byref(f), FAKE, FAKE, cap, FAKE, cap, 0, 0, None)
    assert lib.ds4c_compress_decode_one(*args(1)) == B.DS4C_ECAP
    f.n_index_comp = 0
    assert lib.ds4c_compress_decode_one(*args(10)) == B.DS4C_EPOS
    f.n_index_comp = 1
    assert lib.ds4c_compress_decode_one(ctypes.byref(L), ctypes.byref(f), 0, FAKE, 10, FAKE, 10, 0, 0,
                                        None) == B.DS4C_EINVAL
    assert f.n_tokens == 7


def _blob_header(ratio=4, coff=2, da=512, di=128, n_rot=64, n=10, nc=2, ni=2, magic=0x46345344, version=1):
    return struct.pack("<8I3Q", magic, version, ratio, coff, da, di, n_rot, 0, n, nc, ni)


@pytest.mark.parametrize("kw", [
    dict(magic=0x12345678), dict(version=2), dict(ratio=128), dict(coff=1), dict(da=256),
    dict(di=64), dict(n_rot=32), dict(nc=3), dict(ni=1),
])
def test_load_rejects_bad_blobs(kw):
    L, f = make_layer(), frontier()
    n = B.ds4c_frontier_blob_bytes(L)
    blob = _blob_header(**kw) + b"\0" * (n - 56)
    buf = ctypes.create_string_buffer(blob, len(blob))
    assert B.lib().ds4c_frontier_load(ctypes.byref(L), ctypes.byref(f), buf, len(blob), None) == B.DS4C_EFORMAT
    assert f.n_tokens == 0


def test_load_rejects_wrong_length():
    L, f = make_layer(), frontier()
    n = B.ds4c_frontier_blob_bytes(L)
    for size in (n - 1, n + 1, 55):
        blob = (_blob_header() + b"\0" * n)[:size]
        buf = ctypes.create_string_buffer(blob, len(blob))
        assert B.lib().ds4c_frontier_load(ctypes.byref(L), ctypes.byref(f), buf, len(blob), None) == B.DS4C_EFORMAT


def test_save_rejects_small_buffer():
    L, f = make_layer(), frontier(n=12)
    n = B.ds4c_frontier_blob_bytes(L)
    buf = ctypes.create_string_buffer(n)
    w = ctypes.c_size_t(0)
    assert B.lib().ds4c_frontier_save(ctypes.byref(L), ctypes.byref(f), buf, n - 1, ctypes.byref(w),
                                      None) == B.DS4C_ECAP
    f.n_comp = 0
    assert B.lib().ds4c_frontier_save(ctypes.byref(L), ctypes.byref(f), buf, n, ctypes.byref(w),
                                      None) == B.DS4C_EPOS


def test_profile_read_without_records():
    B.ds4c_profile_enable(True)
    ms, cnt = B.ds4c_profile_read()
    assert ms == [0.0] * B.KCLASS_COUNT and cnt == [0] * B.KCLASS_COUNT
    B.ds4c_profile_enable([B.KCLASS_PROJ, B.KCLASS_CARRY, B.KCLASS_INDEXER])
    ms, cnt = B.ds4c_profile_read()
    assert cnt == [0] * B.KCLASS_COUNT
    B.ds4c_profile_enable(False)


def test_profile_mask_out_of_range():
    assert B.lib().ds4c_profile_enable(-1) == B.DS4C_EINVAL
    assert B.lib().ds4c_profile_enable(B.PROFILE_ALL + 1) == B.DS4C_EINVAL
    assert B.lib().ds4c_profile_enable(0) == B.DS4C_OK


def test_profile_evict_validation():
    """Only the pointer and size are stored; no device call is made."""
    f = B.lib().ds4c_profile_evict
    assert f(None, 16, 0) == B.DS4C_EINVAL
    assert f(ctypes.c_void_p(4096), 0, 0) == B.DS4C_EINVAL
    assert f(ctypes.c_void_p(4104), 4096, 0) == B.DS4C_EINVAL
    assert f(ctypes.c_void_p(4096), 4100, 1) == B.DS4C_EINVAL
    assert f(ctypes.c_void_p(4096), 4096, 2) == B.DS4C_EINVAL
    assert f(ctypes.c_void_p(4096), 1 << 20, 0) == B.DS4C_OK
    assert f(ctypes.c_void_p(4096), 1 << 20, 1) == B.DS4C_OK
    assert f(None, 0, 0) == B.DS4C_OK


def test_mixed_attention_workspace_and_validation():
    """Host-side refusals of the mixed-attention call (no device work)."""
    ws = B.ds4c_mixed_attention_workspace_bytes
    # ceil((128 + 512) / 32) = 20 splits of 64 heads x 512 dims, plus max and sum.
    assert ws(64, 512, 128, 512) == 20 * 64 * 512 * 4 + 2 * 5120
    assert ws(64, 512, 0, 0) > 0
    for bad in [(4, 512, 128, 512), (12, 512, 128, 512), (136, 512, 128, 512), (64, 96, 128, 512),
                (64, 512, -1, 512), (64, 512, 128, 4097), (64, 512, 4097, 8)]:
        assert ws(*bad) == 0, bad
    f = B.lib().ds4c_mixed_attention
    P = ctypes.c_void_p(1 << 20)  # aligned stand-in; every call below is refused before use
    W = ctypes.c_void_p(1 << 24)
    need = ws(64, 512, 128, 512)

    def call(**kw):
        a = dict(q=P, H=64, D=512, ring=P, ring_cap=128, first=0, last=99, window=128, comp=P, n_comp=25,
                 topk=P, k=512, qpos=99, ratio=4, out=P, ws=W, ws_bytes=need)
        a.update(kw)
        return f(a["q"], a["H"], a["D"], a["ring"], a["ring_cap"], a["first"], a["last"], a["window"], a["comp"],
                 a["n_comp"], a["topk"], a["k"], a["qpos"], a["ratio"], a["out"], a["ws"], a["ws_bytes"], None)

    assert call(H=60) == B.DS4C_ESHAPE
    assert call(D=320) == B.DS4C_ESHAPE
    assert call(ratio=0) == B.DS4C_EINVAL
    assert call(qpos=-1) == B.DS4C_EINVAL
    assert call(window=-1) == B.DS4C_EINVAL
    assert call(q=None) == B.DS4C_EINVAL
    assert call(q=ctypes.c_void_p((1 << 20) + 4)) == B.DS4C_EINVAL
    assert call(last=128) == B.DS4C_EINVAL           # 129 held positions in a ring of 128
    assert call(ring=None) == B.DS4C_EINVAL          # raw rows are attended
    assert call(n_comp=24) == B.DS4C_ECAP            # 25 rows visible at qpos 99
    assert call(comp=None) == B.DS4C_EINVAL
    assert call(topk=None) == B.DS4C_EINVAL
    assert call(ws=None) == B.DS4C_EINVAL
    assert call(ws_bytes=need - 1) == B.DS4C_ECAP


def _stack(n=4):
    layers = (B.Layer * n)()
    fronts = (B.Frontier * n)()
    for i in range(n):
        r = B.ds4c_layer_ratio(0, i)
        if r == 0:
            layers[i].ratio = 0
            continue
        layers[i] = make_layer(ratio=r)
        f = frontier(n=0, ratio=r)
        f.state = FAKE + 0x10000000 + i * 0x1000000
        fronts[i] = f
    return layers, fronts


def _stack_call(layers, fronts, T=64, cap=10**6, ws=None, x=FAKE + 0x20000000):
    n = len(layers)
    ar = (ctypes.c_void_p * n)(*[FAKE + 0x30000000 if layers[i].ratio else 0 for i in range(n)])
    ac = (ctypes.c_int64 * n)(*[cap] * n)
    ir = (ctypes.c_void_p * n)(*[FAKE + 0x40000000 if layers[i].ratio == 4 else 0 for i in range(n)])
    ic = (ctypes.c_int64 * n)(*[cap if layers[i].ratio == 4 else 0 for i in range(n)])
    wsb = B.ds4c_stack_workspace_bytes(layers, min(T, 4096) or 1) if ws is None else ws
    return B.lib().ds4c_compress_stack_prefill(layers, n, fronts, x, T, 0, ar, ac, ir, ic,
                                               FAKE + 0x50000000, wsb, None)


def test_stack_workspace_is_the_largest_layer_need():
    layers, _ = _stack(4)  # ratios 0, 0, 4, 128
    assert B.ds4c_stack_workspace_bytes(layers, 4096) == max(
        B.ds4c_workspace_bytes(make_layer(ratio=4), 4096), B.ds4c_workspace_bytes(make_layer(ratio=128), 4096))
    layers[2].ratio = 5
    assert B.ds4c_stack_workspace_bytes(layers, 4096) == 0


def test_stack_prefill_validates_everything_first():
    layers, fronts = _stack(4)
    fronts[3].n_tokens = 128  # ratio-128 layer ahead of the ratio-4 layer
    fronts[3].n_comp = 1
    assert _stack_call(layers, fronts) == B.DS4C_EPOS
    assert fronts[2].n_tokens == 0 and fronts[3].n_tokens == 128
    layers, fronts = _stack(4)
    assert _stack_call(layers, fronts, T=400, cap=99) == B.DS4C_ECAP     # 100 rows needed on the ratio-4 layer
    assert _stack_call(layers, fronts, T=64, ws=1024) == B.DS4C_ECAP
    assert _stack_call(layers, fronts, T=0) == B.DS4C_OK
    layers[3].attn.head_dim = 100
    assert _stack_call(layers, fronts) == B.DS4C_ESHAPE
    for i in range(4):
        assert fronts[i].n_tokens == 0
    # a stack with no compressed layer is a no-op
    none = (B.Layer * 2)()
    nf = (B.Frontier * 2)()
    assert _stack_call(none, nf) == B.DS4C_OK


def test_stack_rejects_layers_with_different_input_rows():
    layers, fronts = _stack(6)  # ratios 0, 0, 4, 128, 4, 128
    layers[5].hidden = 2048
    assert _stack_call(layers, fronts) == B.DS4C_ESHAPE


def _stack_decode(layers, fronts, n_tok=8, cap=10**6, x=FAKE + 0x20000000):
    n = len(layers)
    ar = (ctypes.c_void_p * n)(*[FAKE + 0x30000000 if layers[i].ratio else 0 for i in range(n)])
    ac = (ctypes.c_int64 * n)(*[cap] * n)
    ir = (ctypes.c_void_p * n)(*[FAKE + 0x40000000 if layers[i].ratio == 4 else 0 for i in range(n)])
    ic = (ctypes.c_int64 * n)(*[cap if layers[i].ratio == 4 else 0 for i in range(n)])
    return B.lib().ds4c_compress_stack_decode(layers, n, fronts, x, n_tok, ar, ac, ir, ic, None)


def test_stack_decode_validates_the_whole_run_first():
    layers, fronts = _stack(6)  # ratios 0, 0, 4, 128, 4, 128
    fronts[4].n_tokens = 4
    fronts[4].n_comp = fronts[4].n_index_comp = 1
    assert _stack_decode(layers, fronts) == B.DS4C_EPOS
    layers, fronts = _stack(6)
    # 400 steps from position 0 emit 100 rows on the ratio-4 layers
    assert _stack_decode(layers, fronts, n_tok=400, cap=99) == B.DS4C_ECAP
    assert _stack_decode(layers, fronts, n_tok=-1) == B.DS4C_EINVAL
    assert _stack_decode(layers, fronts, n_tok=0) == B.DS4C_OK
    assert _stack_decode(layers, fronts, x=FAKE + 0x20000004) == B.DS4C_EINVAL  # x not 16-byte aligned
    layers[5].hidden = 2048
    assert _stack_decode(layers, fronts) == B.DS4C_ESHAPE
    for i in range(6):
        assert fronts[i].n_tokens == 0


# --- stack snapshot (the compressor sections of a session payload) -----------

def _snap_header(layers, n):
    L = len(layers)
    hdr = struct.pack("<IIIIQ", 0x53345344, 1, L, 0, n)
    for i in range(L):
        r = layers[i].ratio
        hdr += struct.pack("<IIII", r, layers[i].attn.head_dim if r else 0,
                           layers[i].index.head_dim if r == 4 else 0, layers[i].n_rot if r else 0)
    hdr += struct.pack(f"<{L}I", *[n // layers[i].ratio if layers[i].ratio else 0 for i in range(L)])
    hdr += struct.pack(f"<{L}I", *[n // 4 if layers[i].ratio == 4 else 0 for i in range(L)])
    return hdr


def test_snapshot_bytes_is_header_plus_sections():
    layers, _ = _stack(4)  # ratios 0, 0, 4, 128
    n = 1000
    want = 24 + 16 * 4 + 8 * 4
    want += (n // 4) * 512 * 4 + 2 * 8 * 1024 * 4 + (n // 4) * 128 * 4 + 2 * 8 * 256 * 4  # ratio-4 layer
    want += (n // 128) * 512 * 4 + 2 * 128 * 512 * 4                                     # ratio-128 layer
    assert B.ds4c_stack_snapshot_bytes(layers, n) == want
    assert B.ds4c_stack_snapshot_bytes(layers, -1) == 0
    layers[3].ratio = 7
    assert B.ds4c_stack_snapshot_bytes(layers, n) == 0


def _snap_arrays(layers, cap=10**6):
    n = len(layers)
    ar = (ctypes.c_void_p * n)(*[FAKE + 0x30000000 if layers[i].ratio else 0 for i in range(n)])
    ac = (ctypes.c_int64 * n)(*[cap if layers[i].ratio else 0 for i in range(n)])
    ir = (ctypes.c_void_p * n)(*[FAKE + 0x40000000 if layers[i].ratio == 4 else 0 for i in range(n)])
    ic = (ctypes.c_int64 * n)(*[cap if layers[i].ratio == 4 else 0 for i in range(n)])
    return ar, ac, ir, ic


def test_snapshot_save_refuses_before_copying():
    layers, fronts = _stack(4)
    for i in (2, 3):
        r = layers[i].ratio
        fronts[i].n_tokens, fronts[i].n_comp = 1000, 1000 // r
        fronts[i].n_index_comp = 1000 // 4 if r == 4 else 0
    ar, _, ir, _ = _snap_arrays(layers)
    size = B.ds4c_stack_snapshot_bytes(layers, 1000)
    buf = ctypes.create_string_buffer(size)
    w = ctypes.c_size_t(0)
    # layers at different positions
    fronts[3].n_tokens, fronts[3].n_comp = 1128, 1128 // 128
    assert B.lib().ds4c_stack_snapshot_save(layers, 4, fronts, ar, ir, buf, size, ctypes.byref(w), None) == B.DS4C_EPOS
    fronts[3].n_tokens, fronts[3].n_comp = 1000, 1000 // 128
    # inconsistent counters
    fronts[2].n_comp = 7
    assert B.lib().ds4c_stack_snapshot_save(layers, 4, fronts, ar, ir, buf, size, ctypes.byref(w), None) == B.DS4C_EPOS
    fronts[2].n_comp = 250
    # too small a buffer
    assert B.lib().ds4c_stack_snapshot_save(layers, 4, fronts, ar, ir, buf, size - 1, ctypes.byref(w), None) == B.DS4C_ECAP
    assert w.value == 0


def test_snapshot_load_refuses_mismatches():
    layers, fronts = _stack(4)
    n = 1000
    size = B.ds4c_stack_snapshot_bytes(layers, n)
    good = bytearray(_snap_header(layers, n)) + bytes(size - len(_snap_header(layers, n)))
    ar, ac, ir, ic = _snap_arrays(layers)

    def load(blob, cap=10**6):
        a, c, i, d = _snap_arrays(layers, cap)
        return B.lib().ds4c_stack_snapshot_load(layers, 4, fronts, a, c, i, d, bytes(blob), len(blob), None)

    bad = bytearray(good); bad[0] ^= 1
    assert load(bad) == B.DS4C_EFORMAT                      # magic
    bad = bytearray(good); bad[4] = 2
    assert load(bad) == B.DS4C_EFORMAT                      # version
    bad = bytearray(good); struct.pack_into("<I", bad, 24 + 16 * 2 + 4, 256)
    assert load(bad) == B.DS4C_EFORMAT                      # head dim of layer 2
    bad = bytearray(good); struct.pack_into("<I", bad, 24 + 16 * 4 + 4 * 2, 249)
    assert load(bad) == B.DS4C_EFORMAT                      # row count of layer 2
    assert load(good[:-4]) == B.DS4C_EFORMAT                # length
    assert load(good, cap=10) == B.DS4C_ECAP                # row buffer capacity
    # nothing was written: counters untouched
    assert [fronts[i].n_tokens for i in range(4)] == [0, 0, 0, 0]


# --- indexer scoring and top-k -------------------------------------------------

def test_indexer_workspace_bytes():
    a256 = lambda v: (v + 255) // 256 * 256
    # scores, candidate keys, then 256 bytes of first-digit counts per 64-row block
    assert B.ds4c_indexer_workspace_bytes(16448, 512) == a256(16448 * 4) + a256(1 * 512 * 8) + 257 * 256 + 256
    assert B.ds4c_indexer_workspace_bytes(40000, 512) == a256(40000 * 4) + a256(2 * 512 * 8) + 625 * 256 + 256
    assert B.ds4c_indexer_workspace_bytes(0, 512) == 256
    assert B.ds4c_indexer_workspace_bytes(1 << 20, 512) > 0      # 32 chunks of 32768 x 512 = 16384 keys
    assert B.ds4c_indexer_workspace_bytes((1 << 20) + 1, 512) == 0  # 33 chunks: too many keys
    assert B.ds4c_indexer_workspace_bytes(10, 0) == 0
    assert B.ds4c_indexer_workspace_bytes(10, 513) == 0


def test_indexer_validates_before_launching():
    def call(H=64, Dh=128, n=100, k=16, ws=None, q=FAKE, rows=FAKE + 0x100000, wsp=FAKE + 0x200000):
        wsb = B.ds4c_indexer_workspace_bytes(n, k) if ws is None else ws
        return B.lib().ds4c_indexer_topk(q, FAKE + 0x300000, H, Dh, rows, n, k, FAKE + 0x400000, FAKE + 0x500000,
                                         None, None, wsp, wsb, None)
    assert call(Dh=96) == B.DS4C_ESHAPE
    assert call(H=3) == B.DS4C_ESHAPE
    assert call(H=68) == B.DS4C_ESHAPE
    assert call(k=0) == B.DS4C_EINVAL
    assert call(k=513) == B.DS4C_EINVAL
    assert call(n=(1 << 20) + 1, k=512) == B.DS4C_ESHAPE
    assert call(q=FAKE + 4) == B.DS4C_EINVAL                     # q not 16-byte aligned
    assert call(rows=0) == B.DS4C_EINVAL
    assert call(wsp=FAKE + 16) == B.DS4C_EINVAL                  # workspace not 256-byte aligned
    assert call(ws=B.ds4c_indexer_workspace_bytes(100, 16) - 1) == B.DS4C_ECAP
    assert call(n=0, rows=0) == B.DS4C_OK                        # nothing to score: no launch


def test_indexer_noalloc_validates_before_launching():
    """The allocation-free indexer refuses what ds4c_indexer_topk refuses, and
    calls whose workspace would exceed its fixed scratch (DS4C_ECAP), before
    any device call."""
    def call(H=64, Dh=128, n=100, k=16, q=FAKE, rows=FAKE + 0x100000):
        return B.lib().ds4c_indexer_topk_noalloc(q, FAKE + 0x300000, H, Dh, rows, n, k, FAKE + 0x400000,
                                                 FAKE + 0x500000, None, None, None)
    assert call(Dh=96) == B.DS4C_ESHAPE
    assert call(H=68) == B.DS4C_ESHAPE
    assert call(k=0) == B.DS4C_EINVAL
    assert call(n=(1 << 20) + 1, k=512) == B.DS4C_ESHAPE
    assert call(q=FAKE + 4) == B.DS4C_EINVAL
    assert call(rows=0) == B.DS4C_EINVAL
    assert call(n=0, rows=0) == B.DS4C_OK
    # every call the workspace variant accepts at k = 512 fits the scratch ...
    assert B.ds4c_indexer_workspace_bytes(1 << 20, 512) <= 8519936
    # ... a longer call at a small k does not: 2,000,000 rows need 8 MB of scores and 8 MB of counts
    assert B.ds4c_indexer_workspace_bytes(2_000_000, 1) > 8519936
    assert call(n=2_000_000, k=1) == B.DS4C_ECAP
