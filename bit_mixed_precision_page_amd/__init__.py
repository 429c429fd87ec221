"""2-bit mixed-precision paged KV cache with fused dequantize-in-attention decode.

The compute lives in ``libkvq.so`` (HIP kernels for gfx950 behind a C ABI,
declared in ``include/kvq.h``).  ``kvq`` is the ctypes binding with the same
entry-point names; it loads the library on import and raises if it is missing.
``inputs`` holds the seeded synthetic workloads.
"""
__all__ = ["kvq", "inputs"]
