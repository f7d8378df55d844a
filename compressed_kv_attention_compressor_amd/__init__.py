"""MI355X-native compressed-KV compressor (ds4 / DeepSeek-V4).

The compute lives in ``libds4c.so`` (HIP for gfx950, C ABI in
``include/ds4c.h``); ``binding`` marshals arguments to it and ``layer`` keeps
device tensors for it.  Importing this package loads nothing; the library is
loaded on first use and its absence is an error.
"""

__all__ = ["binding", "layer", "synth", "build"]
