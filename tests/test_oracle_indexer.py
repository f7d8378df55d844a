"""Pins of the oracle's indexer scoring and top-k (oracle/indexer.py).

Each pin checks the oracle against something other than itself: a
pure-Python brute force on tiny inputs, closed forms (one head, ReLU zeroing,
linearity in the head weights, rotation invariance without the codec),
a library sort for the selection, and idempotence of the query codec.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import indexer


def _rng(seed):
    return np.random.default_rng(seed)


def test_brute_force_tiny():
    g = _rng(1)
    H, D, n, k = 3, 32, 9, 4
    q = g.standard_normal((H, D)).astype(np.float32)
    w = g.standard_normal(H).astype(np.float32)
    rows = g.standard_normal((n, D)).astype(np.float32)
    q_hat, s, top = indexer.select(q, w, rows, k)
    # brute force: plain loops over heads, rows and dims
    for j in range(n):
        tot = 0.0
        for h in range(H):
            dot = 0.0
            for d in range(D):
                dot += float(q_hat[h][d]) * float(rows[j][d])
            tot += float(w[h]) * (dot if dot > 0 else 0.0)
        assert abs(tot - s[j]) <= 1e-12 * max(1.0, abs(tot))
    s32 = s.astype(np.float32)
    best = sorted(range(n), key=lambda j: (-float(s32[j]), j))[:k]
    assert list(top) == best


def _brute_qat(q_row):
    """Pure-Python QAT of one head row, independent of oracle/codecs.py: the
    Sylvester Hadamard entry by entry, H[i][j] = (-1)**popcount(i & j)
    (the closed form of the H_2m = [[H, H], [H, -H]] recursion), scaled by
    1/sqrt(n); then E2M1 in blocks of 32, each scaled by the smallest power of
    two that fits its largest magnitude into 6, rounded to the nearest of
    0, .5, 1, 1.5, 2, 3, 4, 6 with ties to the even code."""
    n = len(q_row)
    z = []
    for i in range(n):
        acc = 0.0
        for j in range(n):
            acc += (-1.0 if bin(i & j).count("1") % 2 else 1.0) * float(q_row[j])
        z.append(float(np.float32(acc / math.sqrt(n))))
    grid = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
    out = []
    for b in range(0, n, 32):
        blk = z[b:b + 32]
        amax = max(abs(v) for v in blk)
        k = 0
        if amax > 0:
            k = -300
            while amax > 6.0 * 2.0 ** k:
                k += 1
        for v in blk:
            a = abs(v) / 2.0 ** k
            best = min(range(8), key=lambda c: (abs(a - grid[c]), c % 2))
            out.append(math.copysign(grid[best] * 2.0 ** k, v))
    return out


@pytest.mark.parametrize("dh", [32, 64, 128])
def test_qat_query_matches_brute_force(dh):
    """Pins the query's rotation and FP4 round trip (Part 3 §9): a dropped
    rotation, a wrong Hadamard order or scale, or a wrong codec fails here."""
    g = _rng(11)
    q = g.standard_normal((3, dh)).astype(np.float32)
    q_hat = indexer.qat_query(q)
    for h in range(3):
        want = _brute_qat(q[h])
        # the oracle rounds the rotated value to float32 before its decision,
        # as the brute force does; the float64 rotations differ only in the
        # last bits, so the codes agree except at an exact tie (none here)
        assert np.array_equal(q_hat[h], np.array(want)), (h, np.flatnonzero(q_hat[h] != np.array(want)))
    # planted mistake: the query quantised without its rotation
    unrot = np.stack([oracle.fp4_row_roundtrip(q[h]) for h in range(3)])
    assert not np.array_equal(unrot[0], np.array(_brute_qat(q[0])))


def test_one_head_unit_weight_is_relu_dot():
    g = _rng(2)
    q_hat = g.standard_normal((1, 128))
    rows = g.standard_normal((50, 128))
    s = indexer.scores(q_hat, np.ones(1), rows)
    want = np.array([max(0.0, float(np.dot(q_hat[0], r))) for r in rows])
    assert np.allclose(s, want, rtol=1e-13, atol=0)


def test_relu_zeroes_opposed_rows():
    g = _rng(3)
    q_hat = g.standard_normal((4, 64))
    rows = -np.abs(g.standard_normal((3, 64)))
    q_pos = np.abs(q_hat)
    s = indexer.scores(q_pos, np.array([1.0, 2.0, 0.5, 3.0]), rows)  # every dot product < 0
    assert np.array_equal(s, np.zeros(3))


def test_linear_in_head_weights():
    g = _rng(4)
    q_hat = g.standard_normal((8, 128))
    rows = g.standard_normal((20, 128))
    w1, w2 = g.standard_normal(8), g.standard_normal(8)
    s1, s2 = indexer.scores(q_hat, w1, rows), indexer.scores(q_hat, w2, rows)
    assert np.allclose(indexer.scores(q_hat, w1 + w2, rows), s1 + s2, rtol=1e-12, atol=1e-12)
    assert np.allclose(indexer.scores(q_hat, 2.0 * w1, rows), 2.0 * s1, rtol=1e-13, atol=0)


def test_rotation_invariance_without_codec():
    """<H q / sqrt n, H y / sqrt n> = <q, y>: scoring in the rotated domain (I2)."""
    g = _rng(5)
    q = g.standard_normal(128)
    y = g.standard_normal(128)
    assert abs(float(np.dot(oracle.wht_normalized(q), oracle.wht_normalized(y))) - float(np.dot(q, y))) < 1e-11


def test_query_codec_is_idempotent_and_on_grid():
    g = _rng(6)
    q = g.standard_normal((64, 128)).astype(np.float32)
    q_hat = indexer.qat_query(q)
    for h in range(64):
        assert np.array_equal(oracle.fp4_row_roundtrip(q_hat[h]), q_hat[h])
        # each block of 32 is a power-of-two multiple of the E2M1 grid
        for b in range(0, 128, 32):
            blk = q_hat[h, b:b + 32]
            amax = float(np.max(np.abs(blk)))
            if amax == 0:
                continue
            k = oracle.pow2_block_exponent(amax, oracle.E2M1_MAX)
            scaled = np.abs(blk) / 2.0 ** k
            grid = np.abs(oracle.e2m1_values())
            assert scaled.max() <= oracle.E2M1_MAX
            assert all(np.min(np.abs(v - grid)) == 0 for v in scaled)


def test_topk_matches_stable_sort_and_ties():
    g = _rng(7)
    s = g.standard_normal(1000).astype(np.float32)
    s[100:110] = s[5]  # a run of ties with an earlier row
    top = indexer.topk(s, 64)
    ref = np.argsort(-s.astype(np.float64), kind="stable")[:64]
    assert np.array_equal(top, ref)
    # equal scores: lower index first
    t = indexer.topk(np.zeros(10, dtype=np.float32), 3)
    assert list(t) == [0, 1, 2]
    # fewer rows than k, and no rows
    assert list(indexer.topk(np.array([1.0, 3.0, 2.0], dtype=np.float32), 8)) == [1, 2, 0]
    assert indexer.topk(np.zeros(0, dtype=np.float32), 8).size == 0


@pytest.mark.parametrize("plant", ["no_relu", "w_ignored", "unrotated_query", "ties_high_first"])
def test_planted_mistakes_fail_a_pin(plant):
    """Each plausible mistake changes the result of one of the pins above."""
    g = _rng(8)
    q = g.standard_normal((4, 64)).astype(np.float32)
    w = np.array([1.0, -2.0, 0.5, 3.0])
    rows = g.standard_normal((12, 64)).astype(np.float32)
    q_hat = indexer.qat_query(q)
    good = indexer.scores(q_hat, w, rows)
    if plant == "no_relu":
        bad = w @ (q_hat @ rows.astype(np.float64).T)
        assert not np.allclose(bad, good)
    elif plant == "w_ignored":
        bad = np.maximum(q_hat @ rows.astype(np.float64).T, 0).sum(axis=0)
        assert not np.allclose(bad, good)
    elif plant == "unrotated_query":
        bad = indexer.scores(np.stack([oracle.fp4_row_roundtrip(q[h]) for h in range(4)]), w, rows)
        assert not np.allclose(bad, good)
    else:
        s = np.zeros(6, dtype=np.float32)
        bad = np.argsort(-s, kind="stable")[::-1][:3]
        assert list(bad) != list(indexer.topk(s, 3))
