"""The per-layer KV compressor, written as the per-token recurrence.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).

Part 3 §4 lists what ds4's CPU reference does for every token: project the
hidden state with ``wkv`` (kv candidates) and ``wgate`` (scores), add the
learned absolute position bias (APE) to the scores, store kv and score into
the recurrent state, and at a ratio boundary pool the state into one row by
a per-dimension softmax, RMS-normalise it, rotate its last 64 dims (tail
RoPE, Part 3 §8) and send it through the FP8 round trip (attention lane) or
the Hadamard + FP4 round trip (indexer lane, Part 3 §9).  Part 3 §5 gives
the ratio-4 state: 8 rows of width 2*head_dim, the current window written
to rows 4..7 at ``4 + pos % 4``, the 8 rows pooled at ``(pos+1) % 4 == 0``,
then rows 4..7 copied to rows 0..3.

This file follows that order one token at a time (``push_token``).  A
second, independent formulation (``window_rows``) computes each row straight
from its window of tokens; the two must agree exactly.

Readings taken where the pages are silent (each is one constant or one
line here):

* Lanes.  The ratio-4 "two lanes" of Part 3 §5 are the attention compressor
  and the indexer compressor (Part 3 §2 shows separate ``attn_state_*`` and
  ``index_state_*`` tensors, Part 3 §6 separate indexer compressor tensors).
  Each lane has its own head_dim D and its own state.
* Width 2D for ratio 4.  Rows 0..3 (the previous window's tokens) supply
  columns [0, D) and rows 4..7 (the current window) columns [D, 2D); dim j of
  the output pools those 8 entries.  This is the only layout in which every
  projected column is used and the output is D wide.
* Empty state rows hold kv = 0 and score = -inf (weight zero), so ratio-4
  row 0 pools only its current window.  A dim whose weights sum to zero
  gives 0, as the page's ``denom > 0 ? sum / denom : 0`` does.
* RoPE position of row k is k * ratio (the first position of its window);
  pairs are adjacent dims (2i, 2i+1) of the tail; theta_i = base**(-2i/n_rot);
  angles are formed and evaluated in float64.  No YaRN scaling.
* RMS norm: y = o * w / sqrt(mean(o**2) + eps) over all D dims.
* The projections have no bias; weights are [out, in] row-major.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Tuple

import numpy as np

from .codecs import fp4_row_roundtrip, fp8_row_roundtrip, wht_normalized


@dataclass
class LaneSpec:
    """One compressor lane: ``kind`` is "attn" (FP8 rows) or "index" (QAT rows)."""

    kind: str
    head_dim: int
    wkv: np.ndarray    # [coff*D, hidden]
    wgate: np.ndarray  # [coff*D, hidden]
    ape: np.ndarray    # [ratio, coff*D]
    norm_w: np.ndarray  # [D]


@dataclass
class LayerSpec:
    ratio: int
    hidden: int
    n_rot: int
    rope_base: float
    rms_eps: float
    attn: LaneSpec
    index: Optional[LaneSpec] = None

    @property
    def coff(self) -> int:
        # Part 3 §5: ratio-4 layers keep two 4-row halves, width 2 * head_dim.
        return 2 if self.ratio == 4 else 1

    def lanes(self) -> List[LaneSpec]:
        return [self.attn] + ([self.index] if self.index is not None else [])


@dataclass
class LaneState:
    kv: np.ndarray       # [coff*ratio, coff*D]
    score: np.ndarray    # [coff*ratio, coff*D]
    rows: List[np.ndarray] = field(default_factory=list)      # final rows
    prequant: List[np.ndarray] = field(default_factory=list)  # after RoPE
    pooled: List[np.ndarray] = field(default_factory=list)    # before RMS


@dataclass
class LayerState:
    n_tokens: int
    lanes: Dict[str, LaneState]


def _check(spec: LayerSpec) -> None:
    if spec.ratio not in (4, 128):
        raise ValueError("compress ratio must be 4 or 128")
    if (spec.index is not None) != (spec.ratio == 4):
        raise ValueError("an indexer lane exists exactly on ratio-4 layers")
    for lane in spec.lanes():
        w = spec.coff * lane.head_dim
        assert lane.wkv.shape == (w, spec.hidden)
        assert lane.wgate.shape == (w, spec.hidden)
        assert lane.ape.shape == (spec.ratio, w)
        assert lane.norm_w.shape == (lane.head_dim,)


def new_layer_state(spec: LayerSpec) -> LayerState:
    """Empty state: every row kv = 0, score = -inf; no token seen."""
    _check(spec)
    lanes = {}
    for lane in spec.lanes():
        shape = (spec.coff * spec.ratio, spec.coff * lane.head_dim)
        lanes[lane.kind] = LaneState(
            kv=np.zeros(shape, dtype=np.float64),
            score=np.full(shape, -np.inf, dtype=np.float64),
        )
    return LayerState(n_tokens=0, lanes=lanes)


def project(lane: LaneSpec, x: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """kv = x . Wkv^T and raw score = x . Wgate^T for tokens x [T, hidden].

    float64 matrix products (a library routine); the APE is added per token
    by ``push_token`` since it depends on the absolute position.
    """
    x = np.asarray(x, dtype=np.float64)
    return x @ lane.wkv.astype(np.float64).T, x @ lane.wgate.astype(np.float64).T


def softmax_pool(kv_entries: np.ndarray, score_entries: np.ndarray) -> np.ndarray:
    """Per-dimension softmax pooling over the entries of one window (Part 3 §4).

    ``kv_entries`` and ``score_entries`` are [n_entries, D]; for every dim j:
    m = max_i s[i, j];  w_i = exp(s[i, j] - m);  o_j = sum w_i kv[i, j] / sum w_i,
    and o_j = 0 when the weights sum to zero (every entry empty).
    """
    s = np.asarray(score_entries, dtype=np.float64)
    v = np.asarray(kv_entries, dtype=np.float64)
    m = np.max(s, axis=0)                      # per-dim maximum score
    empty = m == -np.inf                       # every entry of the dim is empty
    w = np.exp(s - np.where(empty, 0.0, m))    # exp(-inf) = 0
    denom = np.sum(w, axis=0)
    num = np.sum(w * v, axis=0)
    ok = denom > 0
    out = np.where(ok, num / np.where(ok, denom, 1.0), 0.0)
    return out


def rms_norm(o: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """y = o * weight / sqrt(mean(o**2) + eps) over the whole row."""
    o = np.asarray(o, dtype=np.float64)
    return o * np.asarray(weight, dtype=np.float64) / math.sqrt(float(np.mean(o * o)) + eps)


def rope_tail(y: np.ndarray, pos: int, n_rot: int, base: float) -> np.ndarray:
    """Rotate the last ``n_rot`` dims of a row by position ``pos`` (Part 3 §8).

    The first head_dim - n_rot dims are left as they are.  Pair i is the
    adjacent pair (n_nope + 2i, n_nope + 2i + 1), rotated by
    pos * base**(-2i / n_rot).
    """
    y = np.array(y, dtype=np.float64, copy=True)
    n_nope = y.size - n_rot
    for i in range(n_rot // 2):
        theta = float(base) ** (-2.0 * i / n_rot)
        ang = float(pos) * theta
        c, s = math.cos(ang), math.sin(ang)
        a, b = y[n_nope + 2 * i], y[n_nope + 2 * i + 1]
        y[n_nope + 2 * i] = a * c - b * s
        y[n_nope + 2 * i + 1] = a * s + b * c
    return y


def finish_row(spec: LayerSpec, lane: LaneSpec, o: np.ndarray, row_index: int):
    """RMS norm -> tail RoPE -> lane codec.  Returns (pre-quant row, final row).

    Attention lane: FP8 round trip on the non-RoPE dims (Part 3 §9).
    Indexer lane: orthonormal Hadamard rotation of the whole row, then the
    FP4 round trip; the row is kept in the rotated basis.
    """
    y = rms_norm(o, lane.norm_w, spec.rms_eps)
    y = rope_tail(y, row_index * spec.ratio, spec.n_rot, spec.rope_base)
    if lane.kind == "attn":
        final = fp8_row_roundtrip(y, lane.head_dim - spec.n_rot)
    else:
        final = fp4_row_roundtrip(wht_normalized(y))
    return y, final


def _window_entries(spec: LayerSpec, kv: np.ndarray, score: np.ndarray, d: int):
    """The (kv, score) entries each output dim pools, from a lane's state rows."""
    if spec.ratio == 4:
        # previous window (rows 0..3) on columns [0, D); current (rows 4..7)
        # on columns [D, 2D).
        ekv = np.concatenate([kv[0:4, 0:d], kv[4:8, d:2 * d]], axis=0)
        esc = np.concatenate([score[0:4, 0:d], score[4:8, d:2 * d]], axis=0)
    else:
        ekv, esc = kv[:, 0:d], score[:, 0:d]
    return ekv, esc


def push_token(spec: LayerSpec, state: LayerState,
               kv_t: Dict[str, np.ndarray], score_t: Dict[str, np.ndarray]) -> None:
    """Advance the recurrence by one token (Part 3 §4, §5).

    ``kv_t[kind]`` / ``score_t[kind]`` are the token's projections for each
    lane (score without APE).  The token's absolute position is
    ``state.n_tokens``.
    """
    p = state.n_tokens
    r = spec.ratio
    for lane in spec.lanes():
        st = state.lanes[lane.kind]
        slot = (spec.coff - 1) * r + p % r
        st.kv[slot, :] = kv_t[lane.kind]
        st.score[slot, :] = score_t[lane.kind] + lane.ape[p % r, :]
        if (p + 1) % r == 0:
            ekv, esc = _window_entries(spec, st.kv, st.score, lane.head_dim)
            o = softmax_pool(ekv, esc)
            pre, final = finish_row(spec, lane, o, p // r)
            st.pooled.append(o)
            st.prequant.append(pre)
            st.rows.append(final)
            if r == 4:
                # Half shift: rows 4..7 are copied to rows 0..3; rows 4..7
                # keep their values (a copy, not a clear).
                st.kv[0:4, :] = st.kv[4:8, :]
                st.score[0:4, :] = st.score[4:8, :]
    state.n_tokens = p + 1


def prefill(spec: LayerSpec, state: LayerState, x: np.ndarray) -> None:
    """Run a chunk of tokens x [T, hidden] through the recurrence."""
    x = np.asarray(x, dtype=np.float64)
    proj = {lane.kind: project(lane, x) for lane in spec.lanes()}
    for t in range(x.shape[0]):
        push_token(spec, state,
                   {k: v[0][t] for k, v in proj.items()},
                   {k: v[1][t] for k, v in proj.items()})


def decode_one(spec: LayerSpec, state: LayerState, x_t: np.ndarray) -> None:
    """One decode token: the same recurrence step with a single hidden state."""
    prefill(spec, state, np.asarray(x_t, dtype=np.float64).reshape(1, -1))


def rows_emitted(n0: int, t: int, ratio: int) -> int:
    """Rows a lane appends when tokens n0 .. n0+t-1 are pushed."""
    return (n0 + t) // ratio - n0 // ratio


def window_rows(spec: LayerSpec, lane: LaneSpec, kv_all: np.ndarray,
                score_all: np.ndarray, ks) -> Tuple[np.ndarray, np.ndarray]:
    """Closed form: rows ``ks`` of a lane straight from their token windows.

    ``kv_all[p]`` / ``score_all[p]`` are the projections (score without APE)
    of the token at absolute position p: arrays indexed by position, or any
    mapping holding at least the tokens of the requested windows.  Row k of a ratio-128 lane pools tokens 128k .. 128k+127
    on columns [0, D).  Row k of a ratio-4 lane pools tokens 4k-4 .. 4k-1 on
    columns [0, D) and tokens 4k .. 4k+3 on columns [D, 2D); tokens before 0
    are empty.  Returns (pre-quant rows, final rows), each [len(ks), D].
    """
    r, d = spec.ratio, lane.head_dim
    pre, fin = [], []
    for k in ks:
        if r == 4:
            toks = list(range(4 * k - 4, 4 * k + 4))
        else:
            toks = list(range(128 * k, 128 * k + 128))
        ekv = np.zeros((len(toks), d))
        esc = np.full((len(toks), d), -np.inf)
        for i, p in enumerate(toks):
            if p < 0:
                continue
            c0 = d if (r == 4 and i >= 4) else 0
            ekv[i] = kv_all[p][c0:c0 + d]
            esc[i] = score_all[p][c0:c0 + d] + lane.ape[p % r, c0:c0 + d]
        o = softmax_pool(ekv, esc)
        y, final = finish_row(spec, lane, o, k)
        pre.append(y)
        fin.append(final)
    return np.array(pre).reshape(len(ks), d), np.array(fin).reshape(len(ks), d)


def live_frontier_rows(ratio: int, n: int) -> List[Tuple[int, int]]:
    """(state row, token position) pairs that hold live data after n tokens.

    With c = n mod ratio and m = n - c: ratio 4 holds tokens m-4 .. m-1 in
    rows 0..3 (once a window has been emitted, m >= 4) and tokens m .. n-1 in
    rows 4 .. 3+c; ratio 128 holds tokens m .. n-1 in rows 0 .. c-1.  Other
    rows are leftovers the recurrence never reads again.
    """
    c = n % ratio
    m = n - c
    out = []
    if ratio == 4:
        if m >= 4:
            out += [(i, m - 4 + i) for i in range(4)]
        out += [(4 + i, m + i) for i in range(c)]
    else:
        out += [(i, m + i) for i in range(c)]
    return out


def canonical_frontier(spec: LayerSpec, state: LayerState):
    """Each lane's state with non-live rows set to (kv 0, score -inf).

    Part 4 §6-§7: saved state is written in logical order and must let the
    compressor continue exactly; rows the recurrence will overwrite before
    reading carry no information, so they are written in one fixed form.
    """
    live = {row for row, _ in live_frontier_rows(spec.ratio, state.n_tokens)}
    out = {}
    for lane in spec.lanes():
        st = state.lanes[lane.kind]
        kv = np.zeros_like(st.kv)
        sc = np.full_like(st.score, -np.inf)
        for row in live:
            kv[row] = st.kv[row]
            sc[row] = st.score[row]
        out[lane.kind] = (kv, sc)
    return out


def frontier_from_tokens(spec: LayerSpec, n: int, kv_all, score_all):
    """Closed form of the canonical state after n tokens (Part 3 §5, Part 4 §7).

    Live row i holds the token live_frontier_rows assigns to it: its full
    W-wide kv and its score plus APE[p % ratio]; every other row is (0, -inf).
    ``kv_all[p]`` / ``score_all[p]`` as for ``window_rows``.
    """
    out = {}
    for lane in spec.lanes():
        shape = (spec.coff * spec.ratio, spec.coff * lane.head_dim)
        kv = np.zeros(shape)
        sc = np.full(shape, -np.inf)
        for row, p in live_frontier_rows(spec.ratio, n):
            kv[row] = kv_all[lane.kind][p]
            sc[row] = score_all[lane.kind][p] + lane.ape[p % spec.ratio]
        out[lane.kind] = (kv, sc)
    return out

