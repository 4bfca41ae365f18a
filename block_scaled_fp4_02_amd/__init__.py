"""NVFP4 block-scaled FP4 quantization and W4A4 GEMM for MI355X (gfx950).

The compute path is the HIP library ``libnvfp4.so`` built from ``csrc/``; the
Python side (``nvfp4``) only marshals torch tensors into its C entry points.
Importing this package does not load the library; ``nvfp4`` does, and fails
loudly when it is missing.
"""

__all__ = ["inputs"]
