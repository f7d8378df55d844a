"""Test-side glue: turn synthetic parameters into oracle specs and GPU layers."""

from __future__ import annotations

import numpy as np

import oracle
from compressed_kv_attention_compressor_amd import synth


def oracle_spec(shape: synth.LayerShape, params: dict) -> oracle.LayerSpec:
    def lane(kind):
        p = params[kind]
        return oracle.LaneSpec(kind=kind, head_dim=p["head_dim"],
                               wkv=p["wkv"].astype(np.float64), wgate=p["wgate"].astype(np.float64),
                               ape=p["ape"].astype(np.float64), norm_w=p["norm_w"].astype(np.float64))
    return oracle.LayerSpec(ratio=shape.ratio, hidden=shape.hidden, n_rot=shape.n_rot,
                            rope_base=shape.rope_base, rms_eps=shape.rms_eps,
                            attn=lane("attn"), index=lane("index") if "index" in params else None)


def tiny_spec(ratio: int, hidden: int, d_attn: int, d_index: int, seed: int = 0,
              random_norm: bool = True) -> oracle.LayerSpec:
    """A small random layer drawn straight from numpy (oracle-only tests)."""
    rng = np.random.default_rng(seed)
    coff = 2 if ratio == 4 else 1

    def lane(kind, d):
        w = coff * d
        return oracle.LaneSpec(kind=kind, head_dim=d,
                               wkv=rng.normal(0, 0.1, (w, hidden)), wgate=rng.normal(0, 0.3, (w, hidden)),
                               ape=rng.normal(0, 0.5, (ratio, w)),
                               norm_w=rng.normal(1, 0.1, d) if random_norm else np.ones(d))
    return oracle.LayerSpec(ratio=ratio, hidden=hidden, n_rot=64, rope_base=160000.0, rms_eps=1e-6,
                            attn=lane("attn", d_attn), index=lane("index", d_index) if ratio == 4 else None)
