"""Chunk-adaptive mixed-precision KV cache on MI355X (gfx950).

The compute path lives in the HIP library ``libmkv.so`` (C ABI declared in
``include/mkv.h``); ``chunk_mixed_precision_amd.mkv`` is the thin ctypes
binding over it.  Importing this package loads nothing: the library is
opened on first use and a missing or unbuilt library raises at that point.
"""
