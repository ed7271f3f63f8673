"""MXFP4 dequantize-and-multiply on MI355X (gfx950).

The compute path is ``libmxfp4.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/mxfp4.h``).  ``gemm_mxfp4_dequant_amd.mxfp4`` is a thin
ctypes binding with the same entry-point names.  Importing this package does
not load the library, so the seeded input generators in ``inputs`` work on a
machine without a GPU.  Every compute call fails loudly if the library is not
built: there is no CPU fallback.
"""
