"""Pins of the oracle's codecs (FP8 E4M3, FP4 E2M1, Hadamard) to the formats' definitions.

Each test checks the oracle against something other than itself: printed
format points (tests/golden/fp_formats.json), torch's float8_e4m3fn cast, the
closed-form E2M1 grid, scipy's Hadamard matrix, or algebraic identities.
"""

import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.linalg import hadamard

import oracle
from oracle import codecs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "fp_formats.json")))


def test_e4m3_printed_points():
    vals = codecs.e4m3_values()
    for code, v in GOLD["e4m3"]["points"]:
        assert vals[code] == v and math.copysign(1, vals[code]) == math.copysign(1, v)
    for code in GOLD["e4m3"]["nan_codes"]:
        assert math.isnan(vals[code])
    finite = vals[~np.isnan(vals)]
    assert finite.max() == GOLD["e4m3"]["max_finite"]
    assert np.min(finite[finite > 0]) == GOLD["e4m3"]["min_subnormal"]


def test_e4m3_all_codes_roundtrip():
    vals = codecs.e4m3_values()
    for code in range(256):
        if math.isnan(vals[code]):
            continue
        assert codecs.e4m3_encode(np.array([vals[code]]))[0] == code


def test_e4m3_matches_torch_cast():
    """10^6 random float32 values in range: codes equal torch's float8_e4m3fn cast (RNE)."""
    rng = np.random.default_rng(1)
    mags = np.exp(rng.uniform(np.log(1e-4), np.log(448.0), 1_000_000)).astype(np.float32)
    v = (mags * rng.choice([-1, 1], mags.size)).astype(np.float32)
    ours = codecs.e4m3_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps -0 for negatives that round to zero; so do we.
    assert np.array_equal(ours, ref)


def test_e4m3_ties_to_even():
    for v, want in GOLD["e4m3_ties_to_even"]:
        got = codecs.e4m3_decode(codecs.e4m3_encode(np.array([v])))[0]
        assert got == want, (v, got, want)


def test_e2m1_grid_and_ties():
    vals = codecs.e2m1_values()
    assert list(vals) == GOLD["e2m1"]["values"]
    for code in range(16):
        assert codecs.e2m1_encode(np.array([vals[code]]))[0] == code or vals[code] == 0.0
    for v, want in GOLD["e2m1"]["ties_to_even"]:
        got = codecs.e2m1_decode(codecs.e2m1_encode(np.array([v])))[0]
        assert got == want, (v, got, want)


def test_pow2_exponent_definition():
    # smallest k with amax <= qmax * 2**k, checked on exact boundaries
    assert codecs.pow2_block_exponent(448.0, 448.0) == 0
    assert codecs.pow2_block_exponent(np.nextafter(448.0, 1e9), 448.0) == 1
    assert codecs.pow2_block_exponent(224.0, 448.0) == -1
    assert codecs.pow2_block_exponent(np.nextafter(224.0, 1e9), 448.0) == 0
    assert codecs.pow2_block_exponent(6.0, 6.0) == 0
    assert codecs.pow2_block_exponent(1.0, 6.0) == -2  # 1 <= 1.5, 1 > 0.75
    assert codecs.pow2_block_exponent(0.0, 6.0) == 0
    rng = np.random.default_rng(2)
    for a in np.exp(rng.uniform(-30, 30, 2000)):
        k = codecs.pow2_block_exponent(a, 448.0)
        assert a <= math.ldexp(448.0, k) and a > math.ldexp(448.0, k - 1)


@pytest.mark.parametrize("scale", [1e-3, 1.0, 37.0, 3e4])
def test_fp8_roundtrip_idempotent(scale):
    rng = np.random.default_rng(3)
    for _ in range(50):
        row = rng.normal(0, scale, 512)
        q = codecs.fp8_row_roundtrip(row, 448)
        assert np.array_equal(codecs.fp8_row_roundtrip(q, 448), q)
        # the RoPE tail is untouched, bit for bit
        assert np.array_equal(q[448:], row[448:])
        # every quantised value is an E4M3 value times its block's power of two
        for b in range(7):
            blk = q[64 * b:64 * b + 64]
            k = codecs.pow2_block_exponent(float(np.max(np.abs(row[64 * b:64 * b + 64].astype(np.float32)))), 448.0)
            assert np.all(np.isin(np.abs(np.ldexp(blk, -k)), codecs.e4m3_values()[:127]))


def test_fp8_error_bound():
    """Relative error of a normal-range value is at most half an E4M3 ulp (2**-4)."""
    rng = np.random.default_rng(4)
    row = rng.normal(0, 1, 448 * 40)
    q = codecs.fp8_row_roundtrip(row, row.size)
    k = np.repeat(codecs.fp8_block_exponents(row, row.size), 64)
    big = np.abs(row) >= np.ldexp(2.0 ** -6, k)
    rel = np.abs(q - row)[big] / np.abs(row)[big]
    assert rel.max() <= 2.0 ** -4 + 1e-7


def test_fp4_roundtrip_idempotent_and_grid():
    rng = np.random.default_rng(5)
    for _ in range(100):
        row = rng.normal(0, rng.uniform(0.01, 10), 128)
        q = codecs.fp4_row_roundtrip(row)
        assert np.array_equal(codecs.fp4_row_roundtrip(q), q)
        for b in range(4):
            k = codecs.fp4_block_exponents(row)[b]
            assert np.all(np.isin(np.abs(np.ldexp(q[32 * b:32 * b + 32], -k)), codecs.e2m1_values()[:8]))
            # the largest magnitude never exceeds 6 * 2**k (no saturation needed)
            assert np.max(np.abs(row[32 * b:32 * b + 32])) <= 6 * 2.0 ** k * (1 + 1e-7)


@pytest.mark.parametrize("n", [1, 2, 4, 64, 128, 256])
def test_hadamard_matches_scipy(n):
    h = codecs.sylvester_hadamard(n)
    assert np.array_equal(h, hadamard(n))
    assert np.array_equal(h @ h.T, n * np.eye(n))


def test_wht_orthonormal():
    rng = np.random.default_rng(6)
    y = rng.normal(0, 1, 128)
    z = codecs.wht_normalized(y)
    assert abs(np.linalg.norm(z) - np.linalg.norm(y)) < 1e-12 * np.linalg.norm(y)
    # involution: H/sqrt(n) is symmetric and orthogonal
    assert np.allclose(codecs.wht_normalized(z), y, rtol=0, atol=1e-13)
    # first output is the scaled sum, second the alternating sum (Sylvester order)
    assert abs(z[0] - y.sum() / math.sqrt(128)) < 1e-12
    assert abs(z[1] - (y[0::2].sum() - y[1::2].sum()) / math.sqrt(128)) < 1e-12
