"""paged_kv_cache_18_amd: PagedAttention decode on one MI355X (gfx950).

The library is ``libpa.so`` (C ABI declared in ``include/pa.h``): a host block
allocator with refcounts and copy-on-write, a KV append kernel with fused
INT4/FP8 quantize-on-write, and a split-K decode attention kernel that gathers
16-token K/V blocks through per-sequence block tables.  ``binding`` is a thin
ctypes layer with the same names; it loads the shared library on first use and
raises if it has not been built (there is no CPU fallback).
"""

__all__ = ["binding", "workloads"]
