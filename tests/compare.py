"""Comparison rules between GPU results and the oracle (test infrastructure).

* Values before any codec (pre-quant rows, the attention RoPE tail, live
  frontier kv/score): |g - o| <= 2e-3 * max(|o|, rms(o over the row)).
* Values after a codec: each block's power-of-two exponent is recomputed from
  both sides' pre-codec values.  Same exponent: the ordered code distance
  must be <= 1.  Different exponents are accepted only when the oracle's
  block maximum lies within 2e-3 (relative) of the boundary between them;
  then the values must agree to one step of the coarser grid.
"""

from __future__ import annotations

import math

import numpy as np

from oracle import codecs

REL_TOL = 2e-3


def check_prequant(g: np.ndarray, o: np.ndarray, what: str, tol: float = REL_TOL) -> float:
    g = np.asarray(g, dtype=np.float64)
    o = np.asarray(o, dtype=np.float64)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    if o.size == 0:
        return 0.0
    o2 = o.reshape(-1, o.shape[-1]) if o.ndim > 1 else o.reshape(1, -1)
    g2 = g.reshape(o2.shape)
    rms = np.sqrt(np.mean(o2 * o2, axis=1, keepdims=True))
    scale = np.maximum(np.abs(o2), rms)
    err = np.abs(g2 - o2) / np.where(scale > 0, scale, 1.0)
    worst = float(np.max(err))
    if not worst <= tol:
        i = np.unravel_index(np.argmax(err), err.shape)
        raise AssertionError(f"{what}: rel err {worst:.3g} > {tol} at {i}: gpu {g2[i]!r} oracle {o2[i]!r}")
    return worst


def _ordered(codes: np.ndarray, sign_bit: int) -> np.ndarray:
    mag = (codes & (sign_bit - 1)).astype(np.int64)
    return np.where(codes & sign_bit, -mag, mag)


def _grid_step(v: np.ndarray, k: int, mbits: int, emin: int) -> np.ndarray:
    a = np.abs(v) / 2.0 ** k
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, emin)
    return 2.0 ** (e - mbits + k)


def check_codec_blocks(g_final: np.ndarray, o_final: np.ndarray, g_pre: np.ndarray, o_pre: np.ndarray,
                       block: int, fmt: str, what: str) -> int:
    """Compare codec outputs block by block; returns the number of straddle blocks."""
    if fmt == "e4m3":
        qmax, enc, sign, mbits, emin = codecs.E4M3_MAX, codecs.e4m3_encode, 0x80, 3, -6
    else:
        qmax, enc, sign, mbits, emin = codecs.E2M1_MAX, codecs.e2m1_encode, 0x8, 1, 0
    g_final = np.asarray(g_final, np.float64)
    o_final = np.asarray(o_final, np.float64)
    straddles = 0
    for r in range(o_final.shape[0]):
        for b0 in range(0, o_final.shape[1], block):
            sl = slice(b0, b0 + block)
            amax_o = float(np.max(np.abs(np.asarray(o_pre[r, sl], np.float32))))
            ko = codecs.pow2_block_exponent(amax_o, qmax)
            if g_pre is not None:
                amax_g = float(np.max(np.abs(np.asarray(g_pre[r, sl], np.float32))))
                kg = codecs.pow2_block_exponent(amax_g, qmax)
            else:
                # No GPU pre-codec values: the GPU exponent is taken to be the
                # oracle's unless the block sits within tolerance of a boundary.
                kg = ko
                for kk in (ko - 1, ko + 1):
                    edge = math.ldexp(qmax, min(kk, ko))
                    if abs(amax_o - edge) <= REL_TOL * edge:
                        kg = kk
            gv, ov = g_final[r, sl], o_final[r, sl]
            if ko == kg:
                dg = _ordered(enc(np.ldexp(gv, -ko)), sign)
                do = _ordered(enc(np.ldexp(ov, -ko)), sign)
                bad = np.abs(dg - do) > 1
                if np.any(bad):
                    j = int(np.argmax(bad))
                    raise AssertionError(f"{what}: row {r} block {b0 // block} dim {j}: gpu {gv[j]!r} "
                                         f"oracle {ov[j]!r} differ by more than one {fmt} code (k={ko})")
            else:
                edge = math.ldexp(qmax, min(ko, kg))
                if abs(amax_o - edge) > REL_TOL * edge:
                    raise AssertionError(f"{what}: row {r} block {b0 // block}: block exponents "
                                         f"{kg} (gpu) vs {ko} (oracle) with amax {amax_o!r} far from {edge!r}")
                straddles += 1
                step = _grid_step(np.maximum(np.abs(gv), np.abs(ov)), max(ko, kg), mbits, emin)
                if np.any(np.abs(gv - ov) > step * (1 + 1e-12)):
                    raise AssertionError(f"{what}: row {r} straddle block {b0 // block} beyond one step")
    return straddles


def check_attn_rows(g_final, o_final, g_pre, o_pre, n_rot: int, what: str = "attn rows") -> int:
    d = o_final.shape[1]
    nq = d - n_rot
    check_prequant(g_final[:, nq:], o_final[:, nq:], what + " (RoPE tail)")
    if nq == 0:
        return 0
    gp = None if g_pre is None else g_pre[:, :nq]
    return check_codec_blocks(g_final[:, :nq], o_final[:, :nq], gp, o_pre[:, :nq], 64, "e4m3", what)


def check_index_rows(g_final, o_final, g_pre, o_pre, what: str = "index rows") -> int:
    """g_pre may be None (no GPU pre-codec rows); see check_codec_blocks."""
    d = o_final.shape[1]
    if g_pre is None:
        zg = None
    else:
        zg = np.stack([codecs.wht_normalized(row) for row in np.asarray(g_pre, np.float64)]) if len(g_pre) else g_pre
    zo = np.stack([codecs.wht_normalized(row) for row in np.asarray(o_pre, np.float64)]) if len(o_pre) else o_pre
    if len(o_final) == 0:
        return 0
    assert zo.shape[1] == d
    return check_codec_blocks(g_final, o_final, zg, zo, 32, "e2m1", what)
