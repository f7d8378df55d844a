"""Row codecs of the compressor: FP8 E4M3, FP4 E2M1 and the Hadamard rotation.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Part 3 §9 says a finished attention row goes through an FP8 (E4M3) round
trip on its non-RoPE dims, and an indexer row through a Hadamard-128
rotation followed by an FP4 activation round trip.  The pages name the
formats and nothing more; the readings below are the plainest ones that
make the round trip exact and idempotent:

* E4M3 is the "fn" variant: bias 7, 3 mantissa bits, no infinities, the
  all-ones code is NaN, largest finite value 448 = 1.75 * 2**8.
* E2M1: bias 1, 1 mantissa bit, values +-{0, .5, 1, 1.5, 2, 3, 4, 6}.
* Values are scaled per block by a power of two, 2**k with the smallest
  integer k such that the block's largest magnitude fits the format's
  largest finite value (so nothing saturates), then rounded to the nearest
  representable value, ties to the even code, then multiplied back.  FP8
  blocks are 64 wide, FP4 blocks 32 wide.
* The rotation is the Sylvester-ordered Hadamard matrix scaled by
  1/sqrt(n), so it is orthonormal; the indexer row stays rotated.

The quantiser takes its decision on float32 inputs: ds4 keeps its rows as
float (Part 3 §2 shows ``float *`` caches), so the oracle rounds a value to
float32 before choosing its code.  Everything after that is exact.

The encoders are written from the formats' definitions (enumerate the
grid, take the nearest point), not from any bit-twiddling recipe, so that
a reader can check them by eye.
"""

from __future__ import annotations

import math

import numpy as np

E4M3_MAX = 448.0
E2M1_MAX = 6.0
FP8_BLOCK = 64
FP4_BLOCK = 32


def e4m3_values() -> np.ndarray:
    """Value of each of the 256 E4M3fn codes (code 0x7f / 0xff -> NaN).

    Code layout s.eeee.mmm.  e == 0 is subnormal: m/8 * 2**-6.  Otherwise
    (1 + m/8) * 2**(e-7).  The pattern e == 15, m == 7 is NaN (no inf).
    """
    out = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 15 and m == 7:
            out[code] = math.nan
        elif e == 0:
            out[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            out[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return out


def e2m1_values() -> np.ndarray:
    """Value of each of the 16 E2M1 codes, layout s.ee.m, bias 1.

    e == 0 is subnormal: m/2.  Otherwise (1 + m/2) * 2**(e-1).
    """
    out = np.empty(16, dtype=np.float64)
    for code in range(16):
        s = -1.0 if code & 0x8 else 1.0
        e = (code >> 1) & 0x3
        m = code & 0x1
        if e == 0:
            out[code] = s * (m / 2.0)
        else:
            out[code] = s * (1.0 + m / 2.0) * 2.0 ** (e - 1)
    return out


def rne_to_grid(v: np.ndarray, grid_pos: np.ndarray) -> np.ndarray:
    """Index into ``grid_pos`` of the value nearest to |v|, ties to even index.

    ``grid_pos`` holds the non-negative finite values of a format in code
    order (which is also increasing value order), so an even index is an
    even code, i.e. a zero mantissa LSB.  |v| must not exceed the last
    grid point (callers scale first).
    """
    a = np.abs(np.asarray(v, dtype=np.float64))
    if np.any(a > grid_pos[-1]):
        raise ValueError("value outside the format's finite range")
    hi = np.searchsorted(grid_pos, a, side="left")  # grid[hi] >= a
    hi = np.minimum(hi, len(grid_pos) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - grid_pos[lo]
    d_hi = grid_pos[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


_E4M3_POS = e4m3_values()[:127]  # codes 0x00..0x7e, increasing
_E2M1_POS = e2m1_values()[:8]


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """E4M3fn code (uint8) nearest to each value, ties to even; |v| <= 448."""
    v = np.asarray(v, dtype=np.float64)
    idx = rne_to_grid(v, _E4M3_POS).astype(np.uint8)
    # Signed zero is kept as the sign of v; a negative value that rounds to
    # zero becomes -0, as IEEE rounding would.
    neg = np.signbit(v)
    return np.where(neg, idx | np.uint8(0x80), idx).astype(np.uint8)


def e4m3_decode(code: np.ndarray) -> np.ndarray:
    return e4m3_values()[np.asarray(code, dtype=np.int64)]


def e2m1_encode(v: np.ndarray) -> np.ndarray:
    """E2M1 code (uint8, low 4 bits) nearest to each value, ties to even."""
    v = np.asarray(v, dtype=np.float64)
    idx = rne_to_grid(v, _E2M1_POS).astype(np.uint8)
    neg = np.signbit(v)
    return np.where(neg, idx | np.uint8(0x8), idx).astype(np.uint8)


def e2m1_decode(code: np.ndarray) -> np.ndarray:
    return e2m1_values()[np.asarray(code, dtype=np.int64)]


def pow2_block_exponent(amax: float, qmax: float) -> int:
    """Smallest integer k with amax <= qmax * 2**k; 0 when amax == 0.

    Written as the definition: start from an estimate and step until the
    exact comparison holds with k and fails with k - 1.
    """
    amax = float(amax)
    if amax == 0.0:
        return 0
    if not math.isfinite(amax):
        raise ValueError("non-finite block maximum")
    k = math.ceil(math.log2(amax / qmax))
    while amax > math.ldexp(qmax, k):
        k += 1
    while amax <= math.ldexp(qmax, k - 1):
        k -= 1
    return k


def _block_roundtrip(v32: np.ndarray, qmax: float, grid_pos: np.ndarray):
    """Scale one block by 2**-k, round to the grid, scale back.

    Returns (dequantised float64 values, codes-as-grid-index-with-sign, k).
    """
    amax = float(np.max(np.abs(v32))) if v32.size else 0.0
    k = pow2_block_exponent(amax, qmax)
    scaled = np.ldexp(v32.astype(np.float64), -k)  # exact: power of two
    idx = rne_to_grid(scaled, grid_pos)
    q = grid_pos[idx] * np.where(np.signbit(scaled), -1.0, 1.0)
    return np.ldexp(q, k), k


def fp8_row_roundtrip(row: np.ndarray, n_quant: int, block: int = FP8_BLOCK) -> np.ndarray:
    """FP8 E4M3 round trip on dims [0, n_quant) of one row (Part 3 §9).

    The first ``n_quant`` dims (the non-RoPE part, head_dim - n_rot) are cut
    into blocks of ``block`` dims; each block is rounded to float32, scaled
    by its power-of-two exponent, rounded to E4M3 and scaled back.  The
    remaining dims (the RoPE tail) are returned unchanged.
    """
    row = np.asarray(row, dtype=np.float64)
    if n_quant % block:
        raise ValueError("non-RoPE width is not a whole number of FP8 blocks")
    out = row.copy()
    for b0 in range(0, n_quant, block):
        v32 = row[b0:b0 + block].astype(np.float32)
        out[b0:b0 + block], _ = _block_roundtrip(v32, E4M3_MAX, _E4M3_POS)
    return out


def fp8_block_exponents(row: np.ndarray, n_quant: int, block: int = FP8_BLOCK) -> np.ndarray:
    """Per-block exponent k the FP8 round trip would use (for comparisons)."""
    row = np.asarray(row, dtype=np.float64)
    ks = []
    for b0 in range(0, n_quant, block):
        v32 = row[b0:b0 + block].astype(np.float32)
        ks.append(pow2_block_exponent(float(np.max(np.abs(v32))), E4M3_MAX))
    return np.array(ks, dtype=np.int64)


def fp4_row_roundtrip(row: np.ndarray, block: int = FP4_BLOCK) -> np.ndarray:
    """FP4 E2M1 round trip over a whole row, blocks of ``block`` dims."""
    row = np.asarray(row, dtype=np.float64)
    if row.size % block:
        raise ValueError("row width is not a whole number of FP4 blocks")
    out = np.empty_like(row)
    for b0 in range(0, row.size, block):
        v32 = row[b0:b0 + block].astype(np.float32)
        out[b0:b0 + block], _ = _block_roundtrip(v32, E2M1_MAX, _E2M1_POS)
    return out


def fp4_block_exponents(row: np.ndarray, block: int = FP4_BLOCK) -> np.ndarray:
    row = np.asarray(row, dtype=np.float64)
    return np.array(
        [pow2_block_exponent(float(np.max(np.abs(row[b:b + block].astype(np.float32)))), E2M1_MAX)
         for b in range(0, row.size, block)],
        dtype=np.int64,
    )


def sylvester_hadamard(n: int) -> np.ndarray:
    """Sylvester-ordered Hadamard matrix: H_1 = [1], H_2m = [[H, H], [H, -H]]."""
    if n < 1 or n & (n - 1):
        raise ValueError("Hadamard order must be a power of two")
    h = np.ones((1, 1), dtype=np.float64)
    while h.shape[0] < n:
        h = np.block([[h, h], [h, -h]])
    return h


def wht_normalized(row: np.ndarray) -> np.ndarray:
    """z = H_n . y / sqrt(n): the orthonormal Walsh-Hadamard rotation."""
    row = np.asarray(row, dtype=np.float64)
    n = row.size
    return sylvester_hadamard(n) @ row / math.sqrt(n)
