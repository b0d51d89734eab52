"""Paged KV-cache decode for MI355X (gfx950).

The computation lives in the HIP library ``libpa.so`` (C ABI in
``include/pa.h``); ``paged_kv_cache_464_amd.pa`` is its Python binding with
the same function names.  Importing this package loads nothing; the first
call into ``pa`` loads the library and raises if it has not been built.
"""

__all__ = ["pa", "build"]
