"""kv_cache_mixed_amd -- packed low-bit KV cache for MI355X (gfx950).

The compute path is the HIP library ``libkvq.so`` (C ABI in include/kvq.h);
``kv_cache_mixed_amd.kvq`` is its thin ctypes binding.  Importing this package
does not load the library; ``kvq.load()`` does, and raises if it is missing.
"""
__all__ = ["kvq", "synth"]
