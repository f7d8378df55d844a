"""Device-resident compressor layer on top of the C ABI.

PyTorch supplies device memory and the stream; every computation happens in
libds4c.so.  A ``CompressorLayer`` owns the layer's weights, its frontier
state and its append-only row buffers (Part 4 §6: rows 0 .. live count are
contiguous), and calls ``ds4c_compress_prefill`` / ``ds4c_compress_decode_one``.
"""

from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

from . import binding as B


def _dev_tensor(a, dtype, device) -> torch.Tensor:
    if isinstance(a, torch.Tensor):
        return a.to(device=device, dtype=dtype).contiguous()
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device, dtype=dtype).contiguous()


class CompressorLayer:
    """One compressed layer: ratio 4 (attention + indexer lanes) or 128 (attention)."""

    def __init__(self, ratio: int, hidden: int, lanes: Dict[str, dict], *, dtype: str = "bf16",
                 n_rot: int = 64, rope_base: float = 160000.0, rms_eps: float = 1e-6,
                 max_tokens: int = 4096, device: str = "cuda"):
        self.device = torch.device(device)
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.ratio = ratio
        self.hidden = hidden
        self.kinds = ["attn"] + (["index"] if ratio == 4 else [])
        self._keep = []  # tensors whose pointers the descriptor holds
        self.layer = B.Layer()
        self.layer.ratio = ratio
        self.layer.hidden = hidden
        self.layer.n_rot = n_rot
        self.layer.in_dtype = B.DS4C_BF16 if dtype == "bf16" else B.DS4C_F32
        self.layer.rope_base = rope_base
        self.layer.rms_eps = rms_eps
        self.head_dim = {}
        for kind in self.kinds:
            p = lanes[kind]
            wkv = _dev_tensor(p["wkv"], self.tdtype, self.device)
            wgate = _dev_tensor(p["wgate"], self.tdtype, self.device)
            ape = _dev_tensor(p["ape"], torch.float32, self.device)
            norm = _dev_tensor(p["norm_w"], torch.float32, self.device)
            self._keep += [wkv, wgate, ape, norm]
            lane = B.Lane(int(p["head_dim"]), wkv.data_ptr(), wgate.data_ptr(), ape.data_ptr(), norm.data_ptr())
            setattr(self.layer, kind, lane)
            self.head_dim[kind] = int(p["head_dim"])
        self.frontier = B.Frontier()
        nbytes = B.ds4c_frontier_bytes(self.layer)
        if nbytes == 0:
            raise B.DS4CError(B.DS4C_EINVAL, "layer descriptor rejected")
        self.state = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        self.frontier.state = self.state.data_ptr()
        self.cap = max_tokens // ratio + 1
        self.rows = {k: torch.empty((self.cap, self.head_dim[k]), dtype=torch.float32, device=self.device)
                     for k in self.kinds}
        self._ws: Optional[torch.Tensor] = None
        self.reset()

    @staticmethod
    def stream() -> int:
        return torch.cuda.current_stream().cuda_stream

    # -- state -----------------------------------------------------------------------------
    def reset(self) -> None:
        """Empty frontier (kv 0, score -inf) and zero counters."""
        B.ds4c_frontier_init(self.layer, self.frontier, self.stream())

    @property
    def n_tokens(self) -> int:
        return self.frontier.n_tokens

    def reserve(self, T: int) -> None:
        need = B.ds4c_workspace_bytes(self.layer, T)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=self.device)

    def live_rows(self, kind: str) -> torch.Tensor:
        n = self.frontier.n_comp if kind == "attn" else self.frontier.n_index_comp
        return self.rows[kind][:n]

    def frontier_views(self):
        """(kv, score) device views of each lane's frontier tensors."""
        out, off = {}, 256
        coff = 2 if self.ratio == 4 else 1
        for kind in self.kinds:
            w = coff * self.head_dim[kind]
            n = coff * self.ratio * w
            f = self.state[off:off + 8 * n].view(torch.float32)
            out[kind] = (f[:n].view(coff * self.ratio, w), f[n:].view(coff * self.ratio, w))
            off += 8 * n
        return out

    # -- compute ------------------------------------------------------------------------------
    def prefill(self, x: torch.Tensor, prequant: bool = False) -> Dict[str, torch.Tensor]:
        """Compress tokens x [T, hidden]; returns the pre-codec rows if asked."""
        assert x.dtype == self.tdtype and x.is_contiguous() and x.shape[1] == self.hidden
        T = x.shape[0]
        self.reserve(T)
        n0 = self.frontier.n_tokens
        n_emit = (n0 + T) // self.ratio - n0 // self.ratio
        pre = {k: torch.empty((max(n_emit, 1), self.head_dim[k]), dtype=torch.float32, device=self.device)
               for k in self.kinds} if prequant else {}
        B.ds4c_compress_prefill(
            self.layer, self.frontier, x.data_ptr(), T,
            self.rows["attn"].data_ptr(), self.cap,
            self.rows["index"].data_ptr() if "index" in self.rows else 0, self.cap if "index" in self.rows else 0,
            self._ws.data_ptr(), self._ws.numel(),
            pre["attn"].data_ptr() if prequant else 0,
            pre["index"].data_ptr() if prequant and "index" in pre else 0,
            self.stream())
        return {k: v[:n_emit] for k, v in pre.items()}

    def decode_one(self, x: torch.Tensor, prequant: bool = False) -> Dict[str, torch.Tensor]:
        assert x.dtype == self.tdtype and x.is_contiguous() and x.numel() == self.hidden
        pos = self.frontier.n_tokens
        n_emit = 1 if (pos + 1) % self.ratio == 0 else 0
        pre = {k: torch.empty((1, self.head_dim[k]), dtype=torch.float32, device=self.device)
               for k in self.kinds} if prequant else {}
        B.ds4c_compress_decode_one(
            self.layer, self.frontier, x.data_ptr(),
            self.rows["attn"].data_ptr(), self.cap,
            self.rows["index"].data_ptr() if "index" in self.rows else 0, self.cap if "index" in self.rows else 0,
            pre["attn"].data_ptr() if prequant else 0,
            pre["index"].data_ptr() if prequant and "index" in pre else 0,
            self.stream())
        return {k: v[:n_emit] for k, v in pre.items()}

    def save(self) -> bytes:
        return B.ds4c_frontier_save(self.layer, self.frontier, self.stream())

    def load(self, blob: bytes) -> None:
        B.ds4c_frontier_load(self.layer, self.frontier, blob, self.stream())


class CompressorStack:
    """A stack of compressed layers driven by the native stack entry points.

    ``layers[l]`` is a CompressorLayer, or None for an uncompressed layer
    (ratio 0).  The chunk and layer loops run inside the library.
    """

    def __init__(self, layers):
        self.layers = list(layers)
        n = len(self.layers)
        self.c_layers = (B.Layer * n)()
        self.c_front = (B.Frontier * n)()
        for i, L in enumerate(self.layers):
            if L is None:
                self.c_layers[i].ratio = 0
            else:
                self.c_layers[i] = L.layer
        self._ws: Optional[torch.Tensor] = None
        self._ws_chunk = 0

    def _check_x(self, x: torch.Tensor, n: int) -> None:
        """The library reads x as n rows of the layers' input dtype and width."""
        L0 = next(L for L in self.layers if L is not None)
        assert x.dtype == L0.tdtype and x.is_contiguous() and x.device.type == L0.device.type, \
            "x: dtype, layout or device"
        assert x.numel() == n * L0.hidden, "x: shape"

    def _arrays(self):
        ar = [L.rows["attn"].data_ptr() if L else 0 for L in self.layers]
        ac = [L.cap if L else 0 for L in self.layers]
        ir = [L.rows["index"].data_ptr() if L and "index" in L.rows else 0 for L in self.layers]
        ic = [L.cap if L and "index" in L.rows else 0 for L in self.layers]
        return ar, ac, ir, ic

    def _push(self):
        for i, L in enumerate(self.layers):
            if L is not None:
                self.c_front[i] = L.frontier

    def _pull(self):
        for i, L in enumerate(self.layers):
            if L is not None:
                f = self.c_front[i]
                L.frontier.n_tokens, L.frontier.n_comp, L.frontier.n_index_comp = f.n_tokens, f.n_comp, f.n_index_comp

    def reserve(self, chunk: int) -> None:
        need = B.ds4c_stack_workspace_bytes(self.c_layers, chunk)
        if self._ws is None or self._ws.numel() < need:
            dev = next(L.device for L in self.layers if L is not None)
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

    def prefill(self, x: torch.Tensor, chunk_cap: int = 0) -> None:
        T = x.shape[0]
        self._check_x(x, T)
        chunk = chunk_cap if chunk_cap > 0 else B.ds4c_prefill_chunk_cap(T, 0)
        self.reserve(min(chunk, max(T, 1)))
        self._push()
        ar, ac, ir, ic = self._arrays()
        try:
            B.ds4c_compress_stack_prefill(self.c_layers, self.c_front, x.data_ptr(), T, chunk, ar, ac, ir, ic,
                                          self._ws.data_ptr(), self._ws.numel(), CompressorLayer.stream())
        finally:
            self._pull()

    def snapshot(self) -> bytearray:
        """The compressor sections of a session payload for the whole stack."""
        self._push()
        ar, _, ir, _ = self._arrays()
        return B.ds4c_stack_snapshot_save(self.c_layers, self.c_front, ar, ir, CompressorLayer.stream())

    def restore(self, blob) -> None:
        """Load a snapshot into this stack's existing rows and frontiers."""
        self._push()
        ar, ac, ir, ic = self._arrays()
        try:
            B.ds4c_stack_snapshot_load(self.c_layers, self.c_front, blob, ar, ac, ir, ic, CompressorLayer.stream())
        finally:
            self._pull()

    def decode_one(self, x: torch.Tensor) -> None:
        self._check_x(x, 1)
        self._push()
        ar, ac, ir, ic = self._arrays()
        try:
            B.ds4c_compress_stack_decode_one(self.c_layers, self.c_front, x.data_ptr(), ar, ac, ir, ic,
                                             CompressorLayer.stream())
        finally:
            self._pull()

    def decode(self, x: torch.Tensor) -> None:
        """x [n, hidden]: n single-token decode steps through the stack, in the library."""
        assert x.dim() == 2
        self._check_x(x, x.shape[0])
        self._push()
        ar, ac, ir, ic = self._arrays()
        try:
            B.ds4c_compress_stack_decode(self.c_layers, self.c_front, x.data_ptr(), x.shape[0], ar, ac, ir, ic,
                                         CompressorLayer.stream())
        finally:
            self._pull()
