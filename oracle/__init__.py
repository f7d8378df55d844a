"""CPU oracle for the ds4 compressed-KV compressor.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this
package.  The product path (the HIP library and its Python binding) never
touches it, and this package imports nothing from the product.

What it computes, and where that is stated.  Two pages of Yoshiya Kato's
Qiita series on the DwarfStar (ds4) DeepSeek-V4 engine are the source:

* "Part 3" = "Metal グラフと圧縮 KV の実装を読む: compressor、indexer、HC、
  tail-only RoPE (第3回/全8回)".  Sections cited: §1 (per-layer compress
  ratio), §3 (4096-token prefill chunks), §4 (the per-token compressor
  recurrence, store-with-APE and the per-dimension softmax pool), §5 (the
  ratio-4 two-lane, 8-row frontier and its half shift), §6 (indexer tensors
  and shape), §8 (tail-only RoPE, compression RoPE base), §9 (FP8 round trip
  for attention rows, Hadamard + FP4 round trip for indexer rows).
* "Part 4" = "KV キャッシュをディスクの一級市民にする: DwarfStar の KVC と
  DSV4 ペイロードを読む (第4回/全8回)".  Sections cited: §5 and §7 (the
  frontier tensors saved with the compressed rows), §6 (state is written in
  logical order).

Everything is float64 NumPy, written as plainly as possible: one token at a
time through the recurrence, one window at a time through the pool.  Where
the pages leave a step open, the reading taken is named in the docstring of
the function that takes it.

Parity status of each function (how it is pinned to something other than
itself) is listed in ``tests/test_oracle_*.py``; every public function here
has at least one such pin.
"""

from .codecs import (  # noqa: F401
    E4M3_MAX,
    E2M1_MAX,
    e4m3_values,
    e2m1_values,
    rne_to_grid,
    e4m3_encode,
    e4m3_decode,
    e2m1_encode,
    e2m1_decode,
    pow2_block_exponent,
    fp8_row_roundtrip,
    fp4_row_roundtrip,
    sylvester_hadamard,
    wht_normalized,
)
from .compressor import (  # noqa: F401
    LaneSpec,
    LayerSpec,
    LaneState,
    LayerState,
    project,
    softmax_pool,
    rms_norm,
    rope_tail,
    finish_row,
    new_layer_state,
    push_token,
    prefill,
    decode_one,
    window_rows,
    live_frontier_rows,
    canonical_frontier,
    frontier_from_tokens,
    rows_emitted,
)
from .schedule import layer_compress_ratio, prefill_chunk_cap  # noqa: F401
from . import indexer  # noqa: F401
from . import mixed_attention  # noqa: F401
