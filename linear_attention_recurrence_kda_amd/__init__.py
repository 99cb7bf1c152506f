"""MI355X-native Kimi Delta Attention (KDA) recurrence.

The compute lives in ``libkda.so`` (hand-written HIP for gfx950 behind a C ABI,
declared in ``include/kda.h``).  ``kda`` is the thin Python binding over it;
importing this package does not load the library, calling into ``kda`` does,
and fails loudly if it is missing.
"""
__all__ = ["kda", "datagen"]
