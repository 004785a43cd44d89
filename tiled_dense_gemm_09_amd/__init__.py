"""Tiled dense GEMM for AMD Instinct MI355X (gfx950).

``C = epilogue(A . B)`` with f16/bf16 inputs and FP32 accumulation, computed
by hand-written HIP kernels behind a C ABI (``include/tg.h``).  The Python
binding in :mod:`tiled_dense_gemm_09_amd.tg` only marshals arguments; every
step of the computation runs in the HIP library.  Import the binding
explicitly; importing the package loads nothing.
"""
