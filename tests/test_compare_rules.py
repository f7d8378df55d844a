"""The GPU-vs-oracle comparison rules (tests/compare.py) must reject rows that
skipped a codec round trip.

These run on the CPU with oracle rows standing in for GPU rows: the oracle's
own final rows must pass, while its pre-codec rows handed in as final rows
(the FP8 round trip skipped), rotated but unquantised indexer rows (the FP4
round trip skipped), unrotated quantised indexer rows and rows moved two
codes away must each fail.
"""

import numpy as np
import pytest

import oracle
from oracle import codecs
from tests import compare
from tests._helpers import tiny_spec


def _rows(ratio, seed=3):
    spec = tiny_spec(ratio, 48, 128, 64, seed=seed)
    st = oracle.new_layer_state(spec)
    x = np.random.default_rng(seed + 100).normal(0, 1, (64 if ratio == 4 else 256, 48))
    oracle.prefill(spec, st, x)
    out = {}
    for kind, ls in st.lanes.items():
        out[kind] = (np.array(ls.rows), np.array(ls.prequant))
    return spec, out


@pytest.mark.parametrize("ratio", [4, 128])
@pytest.mark.parametrize("with_pre", [True, False])
def test_oracle_rows_pass(ratio, with_pre):
    spec, rows = _rows(ratio)
    fin, pre = rows["attn"]
    assert compare.check_attn_rows(fin, fin, pre if with_pre else None, pre, spec.n_rot) == 0
    if ratio == 4:
        fin, pre = rows["index"]
        assert compare.check_index_rows(fin, fin, pre if with_pre else None, pre) == 0


@pytest.mark.parametrize("ratio", [4, 128])
@pytest.mark.parametrize("with_pre", [True, False])
def test_prequant_rows_as_final_fail(ratio, with_pre):
    """A GPU path that skipped the FP8 round trip would hand back its
    pre-codec rows; they are within a code of the oracle's finals but off
    the E4M3 grid."""
    spec, rows = _rows(ratio)
    fin, pre = rows["attn"]
    with pytest.raises(AssertionError, match="not a e4m3 value|not the FP8 round trip"):
        compare.check_attn_rows(pre.astype(np.float32).astype(np.float64), fin,
                                pre if with_pre else None, pre, spec.n_rot)


@pytest.mark.parametrize("with_pre", [True, False])
def test_rotated_unquantised_index_rows_fail(with_pre):
    spec, rows = _rows(4)
    fin, pre = rows["index"]
    rotated = np.stack([codecs.wht_normalized(r) for r in pre]).astype(np.float32).astype(np.float64)
    with pytest.raises(AssertionError, match="not a e2m1 value"):
        compare.check_index_rows(rotated, fin, pre if with_pre else None, pre)


def test_unrotated_quantised_index_rows_fail():
    spec, rows = _rows(4)
    fin, pre = rows["index"]
    unrot = np.stack([codecs.fp4_row_roundtrip(r) for r in pre])
    with pytest.raises(AssertionError):
        compare.check_index_rows(unrot, fin, pre, pre)


def test_one_code_passes_two_codes_fail():
    spec, rows = _rows(4)
    fin, pre = rows["attn"]
    nq = fin.shape[1] - spec.n_rot
    # move one value of row 2 one E4M3 code towards zero, then two codes
    r, j = 2, 5
    k = codecs.pow2_block_exponent(float(np.max(np.abs(pre[r, :64].astype(np.float32)))), codecs.E4M3_MAX)
    code = int(codecs.e4m3_encode(np.ldexp(fin[r, j], -k)))
    assert code & 0x7f >= 3
    for steps, ok in ((1, True), (2, False)):
        g = fin.copy()
        g[r, j] = np.ldexp(float(codecs.e4m3_decode(code - steps)), k)
        # without GPU pre-codec rows only the code distance decides
        if ok:
            compare.check_attn_rows(g, fin, None, pre, spec.n_rot)
        else:
            with pytest.raises(AssertionError, match="more than one e4m3 code"):
                compare.check_attn_rows(g, fin, None, pre, spec.n_rot)
        # with them, the output must be their exact round trip
        with pytest.raises(AssertionError, match="not the FP8 round trip"):
            compare.check_attn_rows(g, fin, pre, pre, spec.n_rot)
    assert nq % 64 == 0


def test_scale_rule_violation_fails():
    """A block quantised with a scale one power of two too large differs only
    where its values fall among E4M3's subnormals; the exact round-trip check
    catches it."""
    spec, rows = _rows(4)
    fin, pre = rows["attn"]
    pre = pre.copy()
    amax = float(np.max(np.abs(pre[0, :64])))
    pre[0, 10:20] = amax * np.linspace(2e-6, 3e-5, 10)    # values among E4M3 subnormals
    fin = fin.copy()
    fin[0, :pre.shape[1] - spec.n_rot] = codecs.fp8_row_roundtrip(pre[0], pre.shape[1] - spec.n_rot)[:-spec.n_rot]
    blk = pre[0, :64].astype(np.float32).astype(np.float64)
    k = codecs.pow2_block_exponent(float(np.max(np.abs(blk))), codecs.E4M3_MAX) + 1
    grid = codecs.e4m3_values()[:127]
    coarse = np.ldexp(grid[codecs.rne_to_grid(np.ldexp(blk, -k), grid)] * np.where(np.signbit(blk), -1, 1), k)
    assert np.any(coarse != fin[0, :64])
    g = fin.copy()
    g[0, :64] = coarse
    with pytest.raises(AssertionError, match="not the FP8 round trip"):
        compare.check_attn_rows(g, fin, pre, pre, spec.n_rot)


def test_straddle_block_is_counted():
    """A block whose maximum sits on an exponent boundary may be quantised at
    either exponent; the other side's choice is accepted and counted."""
    rng = np.random.default_rng(5)
    pre = rng.normal(0, 1, (1, 64))
    pre[0, 3] = codecs.E4M3_MAX * 2.0 ** -6 * (1 + 1e-4)   # just above 448 * 2^-6: k = -5
    o_fin = codecs.fp8_row_roundtrip(pre[0], 64)[None, :]
    g_pre = pre.copy()
    g_pre[0, 3] = codecs.E4M3_MAX * 2.0 ** -6               # exactly on it: k = -6
    g_fin = codecs.fp8_row_roundtrip(g_pre[0], 64)[None, :]
    n = compare.check_codec_blocks(g_fin, o_fin, g_pre, pre, 64, "e4m3", "straddle")
    assert n == 1


def test_tiny_values_follow_the_pre_codec_tolerance():
    """A value far below its row's scale sits where the block's FP8 grid is
    finer than the pre-codec tolerance: a code that quantising a value within
    that tolerance gives is accepted, one beyond it is not."""
    rng = np.random.default_rng(9)
    pre = rng.normal(0, 1, (1, 64))
    pre[0, 0] = 3.0                  # block maximum: exponent -7, codes near 2e-4 are ~2e-6 apart
    pre[0, 7] = -2.0e-4
    o_fin = codecs.fp8_row_roundtrip(pre[0], 64)[None, :]
    k = codecs.pow2_block_exponent(float(np.max(np.abs(pre[0].astype(np.float32)))), codecs.E4M3_MAX)
    rms = float(np.sqrt(np.mean(pre[0] ** 2)))
    for shift, ok in ((0.5e-3 * rms, True), (3e-3 * rms, False)):
        g_pre = pre.copy()
        g_pre[0, 7] += shift
        g_fin = codecs.fp8_row_roundtrip(g_pre[0], 64)[None, :]
        dist = abs(int(codecs.e4m3_encode(np.ldexp(g_fin[0, 7], -k))) - int(codecs.e4m3_encode(np.ldexp(o_fin[0, 7], -k))))
        assert dist > 1                  # more than one code apart either way
        if ok:
            compare.check_codec_blocks(g_fin, o_fin, None, pre, 64, "e4m3", "tiny")
        else:
            with pytest.raises(AssertionError, match="more than one e4m3 code"):
                compare.check_codec_blocks(g_fin, o_fin, None, pre, 64, "e4m3", "tiny")
