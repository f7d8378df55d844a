"""Seeded synthetic inputs for the compressor workloads.

This module only draws numbers.  It holds none of the compressor's
arithmetic; the GPU path and the CPU oracle both consume what it returns.

Generator: ``numpy.random.Generator(PCG64(SeedSequence(seed, spawn_key=
(workload_id, layer, tensor_id, slab))))``.  Tensor ids: 0 = x, 1 = attention
wkv, 2 = attention wgate, 3 = attention APE, 4 = indexer wkv, 5 = indexer
wgate, 6 = indexer APE, 7 = attention norm weight, 8 = indexer norm weight,
9 / 10 / 11 = indexer query heads / head weights / compressed indexer rows
(indexer scoring inputs).
Hidden states are drawn per 4096-token slab so that any token range can be
regenerated without drawing the whole sequence.

bf16 workloads draw in float32 and round to nearest-even bf16; the arrays
returned are float32 holding exactly those bf16 values, so a cast to
``torch.bfloat16`` is exact and both sides see identical bits.

Distributions (the five workloads of the compressor's measurement plan):
x ~ N(0, 1); wkv, wgate ~ N(0, 0.02); APE ~ N(0, 0.1) in float32; norm
weights are ones unless ``random_norm`` asks for N(1, 0.1).
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

SLAB = 4096


@dataclass(frozen=True)
class LayerShape:
    ratio: int
    hidden: int
    d_attn: int
    d_index: int          # 0 when the layer has no indexer lane
    dtype: str            # "f32" or "bf16"
    n_rot: int = 64
    rope_base: float = 160000.0
    rms_eps: float = 1e-6

    @property
    def coff(self) -> int:
        return 2 if self.ratio == 4 else 1


@dataclass(frozen=True)
class Workload:
    wid: int
    name: str
    tokens: int                    # prefill tokens
    layer: Optional[LayerShape]    # single-layer workloads
    n_layers: int = 0              # stack workloads
    chunk: int = 4096
    decode_tokens: int = 0
    variant: int = 0               # stack schedule: 0 Flash, 1 Pro (Part 3 §1)


FLASH_R4 = LayerShape(ratio=4, hidden=4096, d_attn=512, d_index=128, dtype="bf16")
FLASH_R128 = LayerShape(ratio=128, hidden=4096, d_attn=512, d_index=0, dtype="bf16")

WORKLOADS: Dict[str, Workload] = {
    "r4_small": Workload(1, "ratio-4 layer, 64 tokens, hidden 256, head_dim 128/64, fp32",
                         64, LayerShape(ratio=4, hidden=256, d_attn=128, d_index=64, dtype="f32")),
    "r4_flash": Workload(2, "Flash ratio-4 layer, 4096-token chunk, hidden 4096, head_dim 512/128, bf16",
                         4096, FLASH_R4),
    "r128_flash": Workload(3, "ratio-128 layer, 4096-token chunk, hidden 4096, head_dim 512, bf16",
                           4096, FLASH_R128),
    "stack32": Workload(4, "32-layer Flash stack, one 4096-token chunk, hidden 4096",
                        4096, None, n_layers=32),
    "stack32_long": Workload(5, "32-layer Flash stack, 65536 tokens in 16 chunks of 4096, then 256 decode steps",
                             65536, None, n_layers=32, decode_tokens=256),
    # The Pro schedule: layers 0-1 ratio 128, then ratio 4 on even and 128 on
    # odd layers (32 compressed layers); the same Flash layer shapes.
    "stack32_pro": Workload(6, "32-layer Pro-schedule stack, one 4096-token chunk, hidden 4096",
                            4096, None, n_layers=32, variant=1),
    # Indexer scoring + top-512 of one query over the indexer rows a Flash
    # ratio-4 layer holds after the long prompt (65,792 tokens: 16,448 rows),
    # 64 heads of 128 dims.
    "indexer_c5": Workload(7, "indexer top-512 of one query over 16448 rows, 64 heads x 128 dims", 16448, None),
    # Ratio-4 mixed attention of one decode query over the same layer: the
    # 128-token raw sliding window plus the top 512 of its 16,448 compressed
    # attention rows (512 dims), 64 query heads.
    "mixed_attn_c5": Workload(8, "ratio-4 mixed attention of one decode query, 64 heads x 512 dims, 128 raw rows "
                                 "+ top 512 of 16448 compressed rows", 16448, None),
}


def _gen(seed: int, wid: int, layer: int, tensor_id: int, slab: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(seed, spawn_key=(wid, layer, tensor_id, slab))
    return np.random.Generator(np.random.PCG64(ss))


def round_to_bf16(a: np.ndarray) -> np.ndarray:
    """float32 -> nearest-even bf16 value, returned as float32."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def _normal(g: np.random.Generator, shape, std: float, mean: float = 0.0) -> np.ndarray:
    a = g.standard_normal(size=shape, dtype=np.float32)
    return (a * np.float32(std) + np.float32(mean)).astype(np.float32)


def hidden_states(wid: int, hidden: int, start: int, count: int, dtype: str, seed: int = 0) -> np.ndarray:
    """Tokens [start, start+count) of a workload's hidden-state sequence."""
    out = np.empty((count, hidden), dtype=np.float32)
    t = start
    while t < start + count:
        slab = t // SLAB
        base = _normal(_gen(seed, wid, 0, 0, slab), (SLAB, hidden), 1.0)
        lo = t - slab * SLAB
        hi = min(SLAB, start + count - slab * SLAB)
        out[t - start:t - start + (hi - lo)] = base[lo:hi]
        t += hi - lo
    return round_to_bf16(out) if dtype == "bf16" else out


def layer_params(wid: int, layer: int, shape: LayerShape, seed: int = 0,
                 random_norm: bool = False) -> dict:
    """Weights of one layer: per lane wkv, wgate [coff*D, hidden], ape [ratio, coff*D], norm [D]."""
    out = {}
    lanes = [("attn", shape.d_attn, 1)]
    if shape.d_index:
        lanes.append(("index", shape.d_index, 4))
    for kind, d, tid in lanes:
        w = shape.coff * d
        wkv = _normal(_gen(seed, wid, layer, tid), (w, shape.hidden), 0.02)
        wgate = _normal(_gen(seed, wid, layer, tid + 1), (w, shape.hidden), 0.02)
        if shape.dtype == "bf16":
            wkv, wgate = round_to_bf16(wkv), round_to_bf16(wgate)
        ape = _normal(_gen(seed, wid, layer, tid + 2), (shape.ratio, w), 0.1)
        if random_norm:
            norm = _normal(_gen(seed, wid, layer, 7 if kind == "attn" else 8), (d,), 0.1, 1.0)
        else:
            norm = np.ones(d, dtype=np.float32)
        out[kind] = dict(head_dim=d, wkv=wkv, wgate=wgate, ape=ape, norm_w=norm)
    return out


def stack_layer_shape(ratio: int) -> Optional[LayerShape]:
    """Layer shape of a Flash-stack layer with the given compress ratio."""
    if ratio == 4:
        return FLASH_R4
    if ratio == 128:
        return FLASH_R128
    return None


def indexer_inputs(wid: int, n_rows: int, n_heads: int = 64, head_dim: int = 128, seed: int = 0):
    """Inputs of one indexer scoring call: query heads q [H, Dh] ~ N(0, 1),
    head weights [H] ~ N(0, 1/H) and compressed indexer rows [n, Dh] ~ N(0, 1),
    all float32."""
    q = _normal(_gen(seed, wid, 0, 9), (n_heads, head_dim), 1.0)
    w = _normal(_gen(seed, wid, 0, 10), (n_heads,), 1.0 / np.sqrt(n_heads))
    rows = _normal(_gen(seed, wid, 0, 11), (n_rows, head_dim), 1.0)
    return q, w, rows


def mixed_attention_inputs(wid: int, n_comp: int, n_heads: int = 64, head_dim: int = 512, ring_cap: int = 128,
                           k: int = 512, seed: int = 0):
    """Inputs of one mixed-attention call: query heads q [H, D], the raw
    sliding-window ring [ring_cap, D] and compressed attention rows
    [n_comp, D], all ~ N(0, 1) float32, and a top-k list of min(k, n_comp)
    distinct row indices in random order (int32)."""
    q = _normal(_gen(seed, wid, 0, 12), (n_heads, head_dim), 1.0)
    ring = _normal(_gen(seed, wid, 0, 13), (ring_cap, head_dim), 1.0)
    comp = _normal(_gen(seed, wid, 0, 14), (max(n_comp, 1), head_dim), 1.0)[:n_comp]
    topk = _gen(seed, wid, 0, 15).choice(max(n_comp, 1), size=min(k, n_comp), replace=False).astype(np.int32)
    return q, ring, comp, topk
