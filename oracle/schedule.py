"""Per-layer compress ratio and prefill chunk cap.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__``).
"""

from __future__ import annotations


def layer_compress_ratio(layer: int, variant: str = "flash") -> int:
    """Compress ratio of a layer (Part 3 §1, and its two tables).

    Flash: layers 0 and 1 are not compressed (ratio 0); from layer 2 on, even
    layers use ratio 4 and odd layers ratio 128.  Pro: layers 0 and 1 use
    ratio 128, then the same alternation.
    """
    if variant not in ("flash", "pro"):
        raise ValueError("variant must be 'flash' or 'pro'")
    if layer < 2:
        return 0 if variant == "flash" else 128
    return 4 if layer % 2 == 0 else 128


def prefill_chunk_cap(prompt_len: int, override: int = 0) -> int:
    """Largest prefill chunk (Part 3 §3).

    With no override, a prompt longer than 4096 tokens is prefilled in
    chunks of at most 4096; a shorter prompt goes in one piece.  A positive
    override (ds4 reads it from an environment variable) replaces the cap.
    """
    if override > 0:
        return override
    return 4096 if prompt_len > 4096 else max(prompt_len, 1)
