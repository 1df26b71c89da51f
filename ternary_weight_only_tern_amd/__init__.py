"""Packed ternary (W1.58A16) GEMV/GEMM on AMD MI355X (gfx950).

The compute lives in ``libtern.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/tern.h``); ``ternary_weight_only_tern_amd.lib`` is a
thin ctypes binding with the same names.  ``synth`` draws seeded inputs.
"""
