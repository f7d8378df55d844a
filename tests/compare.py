"""Comparison rules between GPU results and the oracle (test infrastructure).

* Values before any codec (pre-quant rows, the attention RoPE tail, live
  frontier kv/score): |g - o| <= 2e-3 * max(|o|, rms(o over the row)).
* Values after a codec: first, every GPU block must be a codec output -- each
  value a point of the format's grid times the block's power of two 2^kg, none
  beyond the format's maximum.  kg comes from the GPU's pre-codec block, or,
  without it, from the GPU block's own maximum.  A value that skipped the
  round trip is off the grid and fails here.  Where the GPU's attention-lane
  pre-codec rows are at hand (they are exactly what the kernel quantised), its
  FP8 output must equal their round trip bit for bit.  Then each block's exponent is
  recomputed from both sides' pre-codec values.  Same exponent: the ordered
  code distance must be <= 1, unless the GPU code is one that quantising a
  value within the pre-codec tolerance of the oracle's pre-codec value gives
  (the grid is finer than that tolerance only for values far below the
  row's scale: a value 1e-4 of the row's rms in a block whose maximum is 3
  has codes 1.6e-5 of the rms apart).  Different exponents are accepted only when the
  oracle's block maximum lies within 2e-3 (relative) of the boundary between
  them; then the values must agree to one step of the coarser grid.
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


def _on_grid(v: np.ndarray, k: int, qmax: float, enc, dec) -> np.ndarray:
    """True where v is exactly a finite grid value of the format times 2**k
    and |v| <= qmax * 2**k (a value that skipped the codec fails)."""
    a = np.ldexp(np.asarray(v, np.float64), -k)          # exact: a power of two
    inside = np.abs(a) <= qmax
    back = dec(enc(np.where(inside, a, 0.0)))
    return inside & (back == a)


def check_codec_outputs(g_final: np.ndarray, g_pre, block: int, fmt: str, what: str) -> None:
    """Every GPU block must be a codec output (see the module docstring)."""
    if fmt == "e4m3":
        qmax, enc, dec = codecs.E4M3_MAX, codecs.e4m3_encode, codecs.e4m3_decode
    else:
        qmax, enc, dec = codecs.E2M1_MAX, codecs.e2m1_encode, codecs.e2m1_decode
    g_final = np.asarray(g_final, np.float64)
    if not np.all(np.isfinite(g_final)):
        raise AssertionError(f"{what}: non-finite codec output")
    for r in range(g_final.shape[0]):
        for b0 in range(0, g_final.shape[1], block):
            sl = slice(b0, b0 + block)
            gv = g_final[r, sl]
            if g_pre is not None:
                # The pre-codec values the test holds may differ from the
                # kernel's own in the last bits (the indexer rows' rotation is
                # recomputed here in float64), so a maximum within 1e-5 of an
                # exponent boundary admits either neighbour.
                amax_pre = float(np.max(np.abs(np.asarray(g_pre[r, sl], np.float32))))
                k0 = codecs.pow2_block_exponent(amax_pre, qmax)
                cands = [k0] + [kk for kk in (k0 - 1, k0 + 1)
                                if amax_pre > 0 and abs(amax_pre - math.ldexp(qmax, min(kk, k0)))
                                <= 1e-5 * math.ldexp(qmax, min(kk, k0))]
            else:
                cands = [codecs.pow2_block_exponent(float(np.max(np.abs(gv))), qmax)]
            oks = [_on_grid(gv, kk, qmax, enc, dec) for kk in cands]
            if not any(np.all(ok) for ok in oks):
                j = int(np.argmin(oks[0]))
                raise AssertionError(f"{what}: row {r} block {b0 // block} dim {j}: gpu value {gv[j]!r} is not "
                                     f"a {fmt} value times 2^{cands[0]} (no codec round trip)")


def check_codec_blocks(g_final: np.ndarray, o_final: np.ndarray, g_pre: np.ndarray, o_pre: np.ndarray,
                       block: int, fmt: str, what: str) -> int:
    """Check that the GPU blocks are codec outputs, then compare them with the
    oracle's block by block; returns the number of straddle blocks."""
    check_codec_outputs(g_final, g_pre, block, fmt, what)
    if fmt == "e4m3":
        qmax, enc, dec, sign, mbits, emin = codecs.E4M3_MAX, codecs.e4m3_encode, codecs.e4m3_decode, 0x80, 3, -6
    else:
        qmax, enc, dec, sign, mbits, emin = codecs.E2M1_MAX, codecs.e2m1_encode, codecs.e2m1_decode, 0x8, 1, 0
    g_final = np.asarray(g_final, np.float64)
    o_final = np.asarray(o_final, np.float64)
    o_pre64 = np.asarray(o_pre, np.float64)
    row_rms = np.sqrt(np.mean(o_pre64 * o_pre64, axis=1)) if o_pre64.size else np.zeros(0)
    straddles = 0
    for r in range(o_final.shape[0]):
        for b0 in range(0, o_final.shape[1], block):
            sl = slice(b0, b0 + block)
            gv, ov = g_final[r, sl], o_final[r, sl]
            amax_o = float(np.max(np.abs(np.asarray(o_pre[r, sl], np.float32))))
            ko = codecs.pow2_block_exponent(amax_o, qmax)
            if g_pre is not None:
                amax_g = float(np.max(np.abs(np.asarray(g_pre[r, sl], np.float32))))
                kg = codecs.pow2_block_exponent(amax_g, qmax)
            else:
                # No GPU pre-codec values: the block's scale is 2^kg or 2^(kg+1)
                # with kg from its own maximum (a maximum that rounded down to
                # half the format's range reads one lower).  The oracle's
                # exponent is the GPU's when the GPU block lies on its grid.
                kg = codecs.pow2_block_exponent(float(np.max(np.abs(gv))), qmax)
                if ko in (kg, kg + 1) and np.all(_on_grid(gv, ko, qmax, enc, dec)):
                    kg = ko
            if ko == kg:
                dg = _ordered(enc(np.ldexp(gv, -ko)), sign)
                do = _ordered(enc(np.ldexp(ov, -ko)), sign)
                # Codes that quantising any value within the pre-codec
                # tolerance of the oracle's pre-codec value gives (the grid is
                # finer than that tolerance only for values far below the
                # row's scale).
                op = np.asarray(o_pre[r, sl], np.float64)
                delta = REL_TOL * np.maximum(np.abs(op), row_rms[r])
                lo = np.clip(np.ldexp(op - delta, -ko), -qmax, qmax)
                hi = np.clip(np.ldexp(op + delta, -ko), -qmax, qmax)
                d_lo, d_hi = _ordered(enc(lo), sign), _ordered(enc(hi), sign)
                bad = (np.abs(dg - do) > 1) & ((dg < d_lo) | (dg > d_hi))
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
    if gp is not None:
        # The attention lane's pre-codec rows are exactly the values the kernel
        # quantised, so its FP8 output must be their round trip, bit for bit:
        # this pins the scale rule and the rounding, not only the grid.
        want = np.stack([codecs.fp8_row_roundtrip(row, nq) for row in np.asarray(gp, np.float64)]) \
            if len(gp) else np.zeros((0, nq))
        got = np.asarray(g_final[:, :nq], np.float64)
        if not np.array_equal(got, want):
            r, j = np.argwhere(got != want)[0]
            raise AssertionError(f"{what}: row {r} dim {j}: gpu {got[r, j]!r} is not the FP8 round trip "
                                 f"{want[r, j]!r} of its own pre-codec value {float(gp[r, j])!r}")
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
