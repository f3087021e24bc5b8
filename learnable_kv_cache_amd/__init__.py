"""LTE sparse-attention layer for AMD MI355X (gfx950).

The compute path is the HIP library ``liblte.so`` behind the C ABI declared in
``include/lte.h``; :mod:`learnable_kv_cache_amd.lte` is its thin ctypes
binding.  Nothing is loaded at import time: the library is opened on first use
and a missing library is an error, never a fallback.
"""
__all__ = ["lte", "synth"]
