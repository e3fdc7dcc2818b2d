"""MI355X (gfx950) dense half-precision GEMM: C = A.B on row-major fp16/bf16
inputs with fp32 accumulation, behind a C-ABI library (``libdhpt_gemm.so``).

The binding is loaded on first use of :mod:`dense_half_precision_tiled_amd.gemm`;
importing the package (or its input generators) does not touch the GPU.
"""
__all__ = ["gemm", "inputs"]
