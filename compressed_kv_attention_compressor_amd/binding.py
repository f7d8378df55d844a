"""ctypes binding of libds4c.so: the same entry points as include/ds4c.h.

Argument marshalling only.  Every step of the compressor runs in the HIP
library; if the library is missing or cannot be loaded, every call raises.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_double, c_float, c_int, c_int32, c_int64, c_size_t, c_void_p

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libds4c.so")

DS4C_OK = 0
DS4C_EINVAL = -1
DS4C_ESHAPE = -2
DS4C_ECAP = -3
DS4C_EPOS = -4
DS4C_EFORMAT = -5
DS4C_EDEVICE = -6
DS4C_F32 = 0
DS4C_BF16 = 1
KCLASS_PROJ, KCLASS_POOL, KCLASS_DECODE, KCLASS_INIT, KCLASS_CARRY, KCLASS_INDEXER, KCLASS_ATTENTION = 0, 1, 2, 3, 4, 5, 6
KCLASS_DECODE_POOL = 7
KCLASS_COUNT = 8
PROFILE_ALL = 0xFF

# Every function the header declares, with (restype, argtypes).
SIGNATURES = {}


class Lane(ctypes.Structure):
    _fields_ = [("head_dim", c_int32), ("wkv", c_void_p), ("wgate", c_void_p),
                ("ape", c_void_p), ("norm_w", c_void_p)]


class Layer(ctypes.Structure):
    _fields_ = [("ratio", c_int32), ("hidden", c_int32), ("n_rot", c_int32), ("in_dtype", c_int32),
                ("rope_base", c_float), ("rms_eps", c_float), ("attn", Lane), ("index", Lane)]


class Frontier(ctypes.Structure):
    _fields_ = [("n_tokens", c_int64), ("n_comp", c_int64), ("n_index_comp", c_int64),
                ("state", c_void_p)]


_LP, _FP = POINTER(Layer), POINTER(Frontier)
SIGNATURES.update({
    "ds4c_frontier_bytes": (c_size_t, [_LP]),
    "ds4c_workspace_bytes": (c_size_t, [_LP, c_int64]),
    "ds4c_frontier_blob_bytes": (c_size_t, [_LP]),
    "ds4c_frontier_init": (c_int, [_LP, _FP, c_void_p]),
    "ds4c_compress_prefill": (c_int, [_LP, _FP, c_void_p, c_int64, c_void_p, c_int64, c_void_p, c_int64,
                                      c_void_p, c_size_t, c_void_p, c_void_p, c_void_p]),
    "ds4c_compress_decode_one": (c_int, [_LP, _FP, c_void_p, c_void_p, c_int64, c_void_p, c_int64,
                                         c_void_p, c_void_p, c_void_p]),
    "ds4c_frontier_save": (c_int, [_LP, _FP, c_void_p, c_size_t, POINTER(c_size_t), c_void_p]),
    "ds4c_frontier_load": (c_int, [_LP, _FP, c_void_p, c_size_t, c_void_p]),
    "ds4c_stack_workspace_bytes": (c_size_t, [_LP, c_int, c_int64]),
    "ds4c_compress_stack_prefill": (c_int, [_LP, c_int, _FP, c_void_p, c_int64, c_int64, POINTER(c_void_p),
                                            POINTER(c_int64), POINTER(c_void_p), POINTER(c_int64), c_void_p,
                                            c_size_t, c_void_p]),
    "ds4c_compress_stack_decode_one": (c_int, [_LP, c_int, _FP, c_void_p, POINTER(c_void_p), POINTER(c_int64),
                                               POINTER(c_void_p), POINTER(c_int64), c_void_p]),
    "ds4c_compress_stack_decode": (c_int, [_LP, c_int, _FP, c_void_p, c_int64, POINTER(c_void_p), POINTER(c_int64),
                                           POINTER(c_void_p), POINTER(c_int64), c_void_p]),
    "ds4c_stack_snapshot_bytes": (c_size_t, [_LP, c_int, c_int64]),
    "ds4c_stack_snapshot_save": (c_int, [_LP, c_int, _FP, POINTER(c_void_p), POINTER(c_void_p), c_void_p, c_size_t,
                                         POINTER(c_size_t), c_void_p]),
    "ds4c_stack_snapshot_load": (c_int, [_LP, c_int, _FP, POINTER(c_void_p), POINTER(c_int64), POINTER(c_void_p),
                                         POINTER(c_int64), c_void_p, c_size_t, c_void_p]),
    "ds4c_indexer_workspace_bytes": (c_size_t, [c_int64, ctypes.c_int32]),
    "ds4c_indexer_topk": (c_int, [c_void_p, c_void_p, ctypes.c_int32, ctypes.c_int32, c_void_p, c_int64,
                                  ctypes.c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                  c_void_p]),
    "ds4c_indexer_topk_noalloc": (c_int, [c_void_p, c_void_p, ctypes.c_int32, ctypes.c_int32, c_void_p, c_int64,
                                          ctypes.c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_void_p]),
    "ds4c_mixed_attention_workspace_bytes": (c_size_t, [ctypes.c_int32, ctypes.c_int32, c_int64, ctypes.c_int32]),
    "ds4c_mixed_attention": (c_int, [c_void_p, ctypes.c_int32, ctypes.c_int32, c_void_p, c_int64, c_int64, c_int64,
                                     c_int64, c_void_p, c_int64, c_void_p, ctypes.c_int32, c_int64, ctypes.c_int32,
                                     c_void_p, c_void_p, c_size_t, c_void_p]),
    "ds4c_layer_ratio": (c_int, [c_int, c_int]),
    "ds4c_prefill_chunk_cap": (c_int64, [c_int64, c_int64]),
    "ds4c_status_str": (ctypes.c_char_p, [c_int]),
    "ds4c_profile_enable": (c_int, [c_int]),
    "ds4c_profile_read": (c_int, [POINTER(c_double), POINTER(c_int64), c_int]),
    "ds4c_profile_evict": (c_int, [c_void_p, c_size_t, c_int]),
})


class DS4CError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_str(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the library once.  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build the HIP library first "
                               "(python -m compressed_kv_attention_compressor_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_str(status: int) -> str:
    return lib().ds4c_status_str(status).decode()


def _ok(status: int, what: str) -> int:
    if status < 0:
        raise DS4CError(status, what)
    return status


def ds4c_frontier_bytes(layer: Layer) -> int:
    return lib().ds4c_frontier_bytes(ctypes.byref(layer))


def ds4c_workspace_bytes(layer: Layer, max_tokens: int) -> int:
    return lib().ds4c_workspace_bytes(ctypes.byref(layer), max_tokens)


def ds4c_frontier_blob_bytes(layer: Layer) -> int:
    return lib().ds4c_frontier_blob_bytes(ctypes.byref(layer))


def ds4c_frontier_init(layer: Layer, frontier: Frontier, stream: int = 0) -> int:
    return _ok(lib().ds4c_frontier_init(ctypes.byref(layer), ctypes.byref(frontier), stream),
               "ds4c_frontier_init")


def ds4c_compress_prefill(layer: Layer, frontier: Frontier, x: int, T: int, attn_rows: int, attn_cap: int,
                          index_rows: int, index_cap: int, workspace: int, ws_bytes: int,
                          attn_prequant: int = 0, index_prequant: int = 0, stream: int = 0) -> int:
    return _ok(lib().ds4c_compress_prefill(ctypes.byref(layer), ctypes.byref(frontier), x, T, attn_rows,
                                           attn_cap, index_rows, index_cap, workspace, ws_bytes,
                                           attn_prequant, index_prequant, stream),
               "ds4c_compress_prefill")


def ds4c_compress_decode_one(layer: Layer, frontier: Frontier, x: int, attn_rows: int, attn_cap: int,
                             index_rows: int, index_cap: int, attn_prequant: int = 0,
                             index_prequant: int = 0, stream: int = 0) -> int:
    return _ok(lib().ds4c_compress_decode_one(ctypes.byref(layer), ctypes.byref(frontier), x, attn_rows,
                                              attn_cap, index_rows, index_cap, attn_prequant,
                                              index_prequant, stream),
               "ds4c_compress_decode_one")


def ds4c_frontier_save(layer: Layer, frontier: Frontier, stream: int = 0) -> bytes:
    n = ds4c_frontier_blob_bytes(layer)
    buf = ctypes.create_string_buffer(n)
    written = c_size_t(0)
    _ok(lib().ds4c_frontier_save(ctypes.byref(layer), ctypes.byref(frontier), buf, n,
                                 ctypes.byref(written), stream), "ds4c_frontier_save")
    return buf.raw[:written.value]


def ds4c_frontier_load(layer: Layer, frontier: Frontier, blob: bytes, stream: int = 0) -> int:
    buf = ctypes.create_string_buffer(bytes(blob), len(blob))
    return _ok(lib().ds4c_frontier_load(ctypes.byref(layer), ctypes.byref(frontier), buf, len(blob), stream),
               "ds4c_frontier_load")


def ds4c_stack_workspace_bytes(layers, chunk_cap: int) -> int:
    """layers: a ctypes array of Layer."""
    return lib().ds4c_stack_workspace_bytes(layers, len(layers), chunk_cap)


def _ptr_arrays(attn_rows, attn_cap, index_rows, index_cap):
    n = len(attn_rows)
    return ((c_void_p * n)(*attn_rows), (c_int64 * n)(*attn_cap),
            (c_void_p * n)(*index_rows), (c_int64 * n)(*index_cap))


def ds4c_compress_stack_prefill(layers, frontiers, x: int, T: int, chunk_cap: int, attn_rows, attn_cap,
                                index_rows, index_cap, workspace: int, ws_bytes: int, stream: int = 0) -> int:
    """layers / frontiers: ctypes arrays; the row arguments: one entry per layer (0 where unused)."""
    ar, ac, ir, ic = _ptr_arrays(attn_rows, attn_cap, index_rows, index_cap)
    return _ok(lib().ds4c_compress_stack_prefill(layers, len(layers), frontiers, x, T, chunk_cap, ar, ac, ir, ic,
                                                 workspace, ws_bytes, stream), "ds4c_compress_stack_prefill")


def ds4c_compress_stack_decode_one(layers, frontiers, x: int, attn_rows, attn_cap, index_rows, index_cap,
                                   stream: int = 0) -> int:
    ar, ac, ir, ic = _ptr_arrays(attn_rows, attn_cap, index_rows, index_cap)
    return _ok(lib().ds4c_compress_stack_decode_one(layers, len(layers), frontiers, x, ar, ac, ir, ic, stream),
               "ds4c_compress_stack_decode_one")


def ds4c_compress_stack_decode(layers, frontiers, x: int, n_tokens: int, attn_rows, attn_cap, index_rows,
                               index_cap, stream: int = 0) -> int:
    """n_tokens decode steps; x points at [n_tokens, hidden]."""
    ar, ac, ir, ic = _ptr_arrays(attn_rows, attn_cap, index_rows, index_cap)
    return _ok(lib().ds4c_compress_stack_decode(layers, len(layers), frontiers, x, n_tokens, ar, ac, ir, ic, stream),
               "ds4c_compress_stack_decode")


def ds4c_stack_snapshot_bytes(layers, n_tokens: int) -> int:
    return lib().ds4c_stack_snapshot_bytes(layers, len(layers), n_tokens)


def _host_ptr(buf):
    """Address of a bytes or bytearray object's data (the object must outlive the call)."""
    if isinstance(buf, bytearray):
        return ctypes.addressof((ctypes.c_char * len(buf)).from_buffer(buf)) if len(buf) else None
    return ctypes.cast(ctypes.c_char_p(buf), c_void_p).value


def ds4c_stack_snapshot_save(layers, frontiers, attn_rows, index_rows, stream: int = 0) -> bytearray:
    """Snapshot of a stack (all compressed layers at one position), written in place into a bytearray."""
    n = next((f.n_tokens for L, f in zip(layers, frontiers) if L.ratio), 0)
    size = ds4c_stack_snapshot_bytes(layers, n)
    if size == 0:
        raise DS4CError(DS4C_EINVAL, "ds4c_stack_snapshot_bytes")
    buf = bytearray(size)
    written = c_size_t(0)
    ar = (c_void_p * len(layers))(*[p or None for p in attn_rows])
    ir = (c_void_p * len(layers))(*[p or None for p in index_rows])
    _ok(lib().ds4c_stack_snapshot_save(layers, len(layers), frontiers, ar, ir, _host_ptr(buf), size,
                                       ctypes.byref(written), stream), "ds4c_stack_snapshot_save")
    return buf


def ds4c_stack_snapshot_load(layers, frontiers, blob, attn_rows, attn_cap, index_rows, index_cap,
                             stream: int = 0) -> int:
    ar, ac, ir, ic = _ptr_arrays(attn_rows, attn_cap, index_rows, index_cap)
    return _ok(lib().ds4c_stack_snapshot_load(layers, len(layers), frontiers, ar, ac, ir, ic, _host_ptr(blob),
                                              len(blob), stream), "ds4c_stack_snapshot_load")


def ds4c_indexer_workspace_bytes(n_rows: int, k: int) -> int:
    return lib().ds4c_indexer_workspace_bytes(n_rows, k)


def ds4c_indexer_topk(q: int, head_w: int, n_heads: int, head_dim: int, rows: int, n_rows: int, k: int,
                      out_idx: int, out_score: int, q_hat: int, scores: int, workspace: int, ws_bytes: int,
                      stream: int = 0) -> int:
    return _ok(lib().ds4c_indexer_topk(q, head_w, n_heads, head_dim, rows or None, n_rows, k, out_idx, out_score,
                                       q_hat or None, scores or None, workspace, ws_bytes, stream),
               "ds4c_indexer_topk")


def ds4c_indexer_topk_noalloc(q: int, head_w: int, n_heads: int, head_dim: int, rows: int, n_rows: int, k: int,
                              out_idx: int, out_score: int, q_hat: int, scores: int, stream: int = 0) -> int:
    """ds4c_indexer_topk on the library's fixed per-device scratch (no workspace)."""
    return _ok(lib().ds4c_indexer_topk_noalloc(q, head_w, n_heads, head_dim, rows or None, n_rows, k, out_idx,
                                               out_score, q_hat or None, scores or None, stream),
               "ds4c_indexer_topk_noalloc")


def ds4c_layer_ratio(variant: int, layer: int) -> int:
    return lib().ds4c_layer_ratio(variant, layer)


def ds4c_prefill_chunk_cap(prompt_len: int, override_cap: int = 0) -> int:
    return lib().ds4c_prefill_chunk_cap(prompt_len, override_cap)


def ds4c_profile_enable(classes=True) -> None:
    """Time kernels of the given classes: True = all, False = none, or an
    iterable of KCLASS_* values."""
    if classes is True:
        mask = PROFILE_ALL
    elif classes is False or classes is None:
        mask = 0
    else:
        mask = 0
        for c in classes:
            mask |= 1 << int(c)
    _ok(lib().ds4c_profile_enable(mask), "ds4c_profile_enable")


def ds4c_profile_read():
    """(ms[KCLASS_COUNT], count[KCLASS_COUNT]) accumulated per kernel class since the last read."""
    ms = (c_double * KCLASS_COUNT)()
    cnt = (c_int64 * KCLASS_COUNT)()
    _ok(lib().ds4c_profile_read(ms, cnt, KCLASS_COUNT), "ds4c_profile_read")
    return list(ms), list(cnt)


def ds4c_profile_evict(scratch: int = 0, nbytes: int = 0, write: bool = False) -> None:
    """Cold pool timings: while set (a device pointer and its size), timed
    prefill calls read (or, with write, overwrite) the buffer between
    projection and pooling.  (0, 0) turns it off."""
    _ok(lib().ds4c_profile_evict(scratch or None, nbytes, int(write)), "ds4c_profile_evict")


def ds4c_mixed_attention_workspace_bytes(n_heads: int, head_dim: int, ring_cap: int, k: int) -> int:
    return lib().ds4c_mixed_attention_workspace_bytes(n_heads, head_dim, ring_cap, k)


def ds4c_mixed_attention(q, raw_ring, first_raw_pos: int, raw_last_pos: int, window: int, comp_rows, topk,
                         qpos: int, ratio: int, out, workspace, stream: int = 0) -> None:
    """Ratio-4 indexed mixed attention of one decode query (Part 3 §7).
    q [H, D], raw_ring [ring_cap, D], comp_rows [n, D], out [H, D]: float32
    device tensors; topk int32 device tensor [k]; workspace uint8 device
    tensor of ds4c_mixed_attention_workspace_bytes bytes."""
    H, D = q.shape
    _ok(lib().ds4c_mixed_attention(q.data_ptr(), H, D, raw_ring.data_ptr(), raw_ring.shape[0], first_raw_pos,
                                   raw_last_pos, window, comp_rows.data_ptr() if comp_rows.numel() else None,
                                   comp_rows.shape[0], topk.data_ptr() if topk.numel() else None, topk.numel(),
                                   qpos, ratio, out.data_ptr(), workspace.data_ptr(), workspace.numel(),
                                   stream or None),
        "ds4c_mixed_attention")
