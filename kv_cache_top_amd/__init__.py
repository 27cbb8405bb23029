"""ParisKV decode-time KV-cache retrieval for AMD Instinct MI355X (gfx950).

The path lives in libpariskv.so (HIP kernels behind the C ABI of
include/pariskv.h); ``kv_cache_top_amd.pariskv`` is its ctypes binding and
``kv_cache_top_amd.build`` compiles it in-tree.
"""
