"""Ratio-4 indexed mixed attention of one decode query.

TEST INFRASTRUCTURE ONLY (see the package docstring): only tests/, smoke()
and bench.py's cpu_baseline may call this.

What the pages fix (Part 3 §7, with the raw window of Part 3 §2): on ratio-4
layers one attention pass covers two sets of rows.
* Raw rows: the layer keeps the raw KV rows of the latest tokens in a
  sliding window (Flash: 128 tokens).  For a query at position qpos the
  pass covers the raw positions from max(first held position, qpos + 1 -
  window) (or from 0 when the window is 0 or not yet full) through
  min(qpos, last held position).
* Compressed rows: the indexer's top-k list is walked in order; a negative
  entry is skipped and the first entry at or beyond the number of visible
  compressed rows ends the walk.
Both sets feed one online softmax (running max and sum), so the result is
one softmax over their union.

Readings taken where the pages give no formula:

* A1 -- each row is both key and value, shared by every query head: the
  compressor emits one row per position, not one per head.
* A2 -- the logit of head h for row j is <q_h, row_j> / sqrt(D).
* A3 -- visible compressed rows at qpos: floor((qpos + 1) / ratio), the rows
  the compressor has emitted once token qpos is in (its emit count).
* A4 -- the raw ring holds position p at ring row p mod ring_cap.
* A5 -- an index listed twice is attended twice (the walk has no
  de-duplication); the indexer's own lists hold distinct rows.
* A6 -- no sink logit and no output projection; a query with no row to
  attend gets the zero vector.
"""

from __future__ import annotations

import numpy as np


def attended_rows(raw_ring: np.ndarray, first_raw_pos: int, raw_last_pos: int, window: int, comp: np.ndarray,
                  topk, qpos: int, ratio: int = 4) -> np.ndarray:
    """The rows one query attends, raw rows first (ascending position), then
    the compressed rows in list order (Part 3 §7; A3-A5)."""
    ring_cap = raw_ring.shape[0]
    window_first = qpos + 1 - window if (window != 0 and qpos + 1 > window) else 0
    first = max(first_raw_pos, window_first)
    last = min(qpos, raw_last_pos)
    rows = [raw_ring[p % ring_cap] for p in range(first, last + 1)]
    visible = (qpos + 1) // ratio
    for idx in topk:
        idx = int(idx)
        if idx < 0:
            continue
        if idx >= visible:
            break
        rows.append(comp[idx])
    D = raw_ring.shape[1]
    return np.asarray(rows, dtype=np.float64).reshape(len(rows), D)


def attend(q: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """softmax(q rows^T / sqrt(D)) rows for every head (A1, A2, A6), float64."""
    q = np.asarray(q, dtype=np.float64)
    H, D = q.shape
    if rows.shape[0] == 0:
        return np.zeros((H, D))
    logits = q @ rows.T / np.sqrt(D)
    logits -= logits.max(axis=1, keepdims=True)
    p = np.exp(logits)
    p /= p.sum(axis=1, keepdims=True)
    return p @ rows


def mixed_attention(q, raw_ring, first_raw_pos, raw_last_pos, window, comp, topk, qpos, ratio=4) -> np.ndarray:
    """Output [H, D] of one decode query (Part 3 §7)."""
    rows = attended_rows(np.asarray(raw_ring), first_raw_pos, raw_last_pos, window, np.asarray(comp), topk, qpos,
                         ratio)
    return attend(q, rows)
