"""Calibrated FP8 E4M3 paged KV attention for MI355X (gfx950).

The compute lives in ``libkvfp8.so`` (hand-written HIP kernels behind a C ABI
declared in ``include/kvfp8.h``); ``kvfp8`` is its Python binding. Importing
``fp8_quantised_paged_amd.kvfp8`` fails if the library has not been built.
"""

__all__ = ["kvfp8"]
