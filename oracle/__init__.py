"""CPU oracle for the KIVI 2-bit KV cache: test infrastructure only.

Only tests/, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product library never loads it.
"""
