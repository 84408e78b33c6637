"""KIVI 2-bit KV cache for AMD Instinct MI355X (gfx950).

The product is libkivi.so (HIP kernels behind the C ABI in include/kivi.h);
``kv_cache_bit_quantize_amd.kivi`` is its Python binding and ``synth`` the seeded
synthetic workload generator.  Import the binding explicitly:

    from kv_cache_bit_quantize_amd import kivi
"""
