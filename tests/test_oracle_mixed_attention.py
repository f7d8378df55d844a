"""Pins of oracle.mixed_attention (Part 3 §7) to things other than itself:
the row walk against hand-written row lists, softmax attention against
torch's scaled-dot-product attention (a library routine with the 1/sqrt(D)
scale), and closed forms (uniform weights, one row, a dominant row)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import mixed_attention as MA

D = 64


def _rows(n, seed):
    return np.random.default_rng(seed).standard_normal((n, D))


def test_walk_skips_negative_and_stops_at_first_invisible():
    comp = _rows(10, 1)
    ring = _rows(8, 2)
    # qpos 11 -> 3 visible compressed rows; raw: none held (first > last).
    got = MA.attended_rows(ring, 5, 4, 8, comp, [2, -1, 0, 3, 1], 11, 4)
    np.testing.assert_array_equal(got, comp[[2, 0]])
    got = MA.attended_rows(ring, 5, 4, 8, comp, [-1, -7, 1, 1], 11, 4)
    np.testing.assert_array_equal(got, comp[[1, 1]])
    assert MA.attended_rows(ring, 5, 4, 8, comp, [3, 0], 11, 4).shape == (0, D)
    # qpos 2: no compressed row is visible yet.
    assert MA.attended_rows(ring, 5, 4, 8, comp, [0], 2, 4).shape == (0, D)


def test_raw_window_and_ring_rows():
    ring = _rows(8, 3)
    comp = _rows(4, 4)
    # Ring of 8 holds positions 13..20 (p at row p % 8); window 5 at qpos 20
    # covers 16..20; the list adds compressed row 1 (5 visible).
    got = MA.attended_rows(ring, 13, 20, 5, comp, [1], 20, 4)
    np.testing.assert_array_equal(got, np.vstack([ring[[0, 1, 2, 3, 4]], comp[[1]]]))
    # Window 0: every held position up to qpos (here 13..18).
    got = MA.attended_rows(ring, 13, 20, 0, comp, [], 18, 4)
    np.testing.assert_array_equal(got, ring[[5, 6, 7, 0, 1, 2]])
    # Window larger than qpos + 1 starts at position 0 (clipped to what is held).
    got = MA.attended_rows(ring, 0, 3, 100, comp, [], 3, 4)
    np.testing.assert_array_equal(got, ring[[0, 1, 2, 3]])
    # Ratio 128 visibility.
    assert MA.attended_rows(ring, 5, 4, 8, comp, [0], 126, 128).shape == (0, D)
    assert MA.attended_rows(ring, 5, 4, 8, comp, [0], 127, 128).shape == (1, D)


def test_attend_matches_torch_sdpa():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((8, D))
    rows = rng.standard_normal((37, D))
    qt = torch.from_numpy(q).reshape(8, 1, D)            # heads as batch, one query each
    kt = torch.from_numpy(rows).expand(8, 37, D)
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, kt).reshape(8, D).numpy()
    np.testing.assert_allclose(MA.attend(q, rows), ref, rtol=1e-12, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(6)
    rows = rng.standard_normal((9, D))
    # Zero query: uniform weights, the mean row, for every head.
    out = MA.attend(np.zeros((4, D)), rows)
    np.testing.assert_allclose(out, np.tile(rows.mean(axis=0), (4, 1)), rtol=0, atol=1e-14)
    # One row: that row, whatever the query.
    out = MA.attend(rng.standard_normal((4, D)), rows[:1])
    np.testing.assert_allclose(out, np.tile(rows[0], (4, 1)), rtol=0, atol=1e-14)
    # No row: zeros (A6).
    assert not MA.attend(rng.standard_normal((2, D)), rows[:0]).any()
    # A query aligned with one row by a large factor: the weight left for the
    # others is at most n * exp(-gap), so the output is that row within it.
    q = 40.0 * rows[3][None, :] / np.linalg.norm(rows[3])
    logits = (q @ rows.T / np.sqrt(D))[0]
    gap = logits[3] - np.max(np.delete(logits, 3))
    bound = len(rows) * np.exp(-gap) * 2 * np.abs(rows).max()
    assert gap > 5
    np.testing.assert_allclose(MA.attend(q, rows)[0], rows[3], rtol=0, atol=bound)


def test_order_of_the_walk_does_not_change_the_output():
    rng = np.random.default_rng(7)
    ring, comp = _rows(16, 8), _rows(40, 9)
    q = rng.standard_normal((4, D))
    topk = rng.choice(40, size=12, replace=False)
    a = MA.mixed_attention(q, ring, 100, 115, 100, comp, topk, 170, 4)
    b = MA.mixed_attention(q, ring, 100, 115, 100, comp, topk[::-1], 170, 4)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)
    # A duplicated entry counts twice: with a zero query the output is the
    # mean over the walk, duplicate included.
    rows = MA.attended_rows(ring, 100, 115, 100, comp, [4, 4, 9], 170, 4)
    assert rows.shape[0] == 16 + 3
    out = MA.mixed_attention(np.zeros((2, D)), ring, 100, 115, 100, comp, [4, 4, 9], 170, 4)
    exp = (ring.sum(axis=0) + 2 * comp[4] + comp[9]) / 19
    np.testing.assert_allclose(out[0], exp, rtol=0, atol=1e-13)


def test_package_exports_the_module():
    assert oracle.mixed_attention is MA
