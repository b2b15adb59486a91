"""Block-scaled FP4 (MXFP4 / NVFP4 / E4M3-scaled) quantize-dequantize for
AMD MI355X (gfx950): hand-written HIP kernels behind the C ABI of
include/fp4q.h, with a thin ctypes binding (``fp4q``) that marshals torch
tensors to device pointers and streams.

Importing the package loads nothing; the HIP library is loaded on the first
call and a missing build raises an error (there is no CPU fallback).
"""
