"""Indexer scoring and top-k selection over a layer's compressed indexer rows.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests/, smoke()
and bench.py's cpu_baseline may call this.

What the pages fix (Part 3 §6, §9): ratio-4 layers carry an indexer that
scores the compressed indexer rows and hands the attention only the top-k of
them (Flash: 64 indexer heads of 128 dims, top-k 512; the decode kernel keeps
one compressed row per threadgroup and walks the 64 heads in groups of 4).
The indexer's query passes the same QAT round trip as the compressed indexer
rows (Hadamard 128 + FP4); without it the selection would not follow the
model's graph.

Readings taken where the pages give no formula:

* I1 -- score of row j for one query token:
  s_j = sum_h w_h * max(0, <qhat_h, k_j>), where qhat_h is head h's query
  after the QAT round trip and w_h is the token's weight for head h (the
  per-head output of the indexer's projection).  This is the lightning
  indexer of DeepSeek's sparse attention, the plainest form consistent with
  per-head queries and a projection that gives one weight per head.
* I2 -- the dot product is taken in the rotated domain: the rows are stored
  rotated (Hadamard, not inverted) and the query is rotated the same way;
  the rotation is orthonormal, so without the codec the score equals the
  unrotated one.
* I3 -- top-k: the k rows with the largest scores in descending order; equal
  scores go to the lower row index first; with fewer than k rows, all rows.
* I4 -- the selection is decided on float32 scores (the precision the
  kernels produce), so both sides order the same numbers.

Parity unpinned against ds4 itself: no page prints an indexer score.
"""

from __future__ import annotations

import numpy as np

from .codecs import fp4_row_roundtrip, wht_normalized


def qat_query(q: np.ndarray) -> np.ndarray:
    """QAT round trip of every head row of q [H, Dh] (Part 3 §9): the
    orthonormal Hadamard rotation of the row, then FP4 E2M1 in blocks of 32
    with a power-of-two scale; the result stays rotated (I2)."""
    q = np.asarray(q, dtype=np.float64)
    return np.stack([fp4_row_roundtrip(wht_normalized(q[h])) for h in range(q.shape[0])])


def scores(q_hat: np.ndarray, head_w: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """s_j = sum_h w_h * relu(<q_hat_h, rows_j>) for every row (I1), float64."""
    q_hat = np.asarray(q_hat, dtype=np.float64)
    rows = np.asarray(rows, dtype=np.float64)
    head_w = np.asarray(head_w, dtype=np.float64)
    dots = q_hat @ rows.T                      # [H, n]
    return head_w @ np.maximum(dots, 0.0)      # [n]


def topk(s32: np.ndarray, k: int) -> np.ndarray:
    """Row indices of the k largest scores, descending, ties to the lower
    index (I3); the scores are float32 (I4)."""
    s32 = np.asarray(s32, dtype=np.float32)
    n = s32.size
    order = np.lexsort((np.arange(n), -s32.astype(np.float64)))
    return order[:min(k, n)].astype(np.int64)


def select(q: np.ndarray, head_w: np.ndarray, rows: np.ndarray, k: int):
    """The whole step: (q_hat, float64 scores, top-k indices of the float32 scores)."""
    q_hat = qat_query(q)
    s = scores(q_hat, head_w, rows)
    return q_hat, s, topk(s.astype(np.float32), k)
