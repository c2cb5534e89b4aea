"""MI355X-native GEMM, C = alpha*A*B + beta*C, behind a small C-ABI library.

The compute path is ``libgemm.so`` (hand-written HIP kernels for gfx950);
``gemm`` below only marshals torch tensors into that library's C calls.
Importing this package does not load the library; the first call does, and
fails loudly when it has not been built.
"""
from .binding import (  # noqa: F401
    GemmError,
    gemm,
    gemm_bf16,
    gemm_f32,
    gemm_naive_bf16,
    gemm_naive_f32,
    last_kernel,
    library,
    library_path,
)

__all__ = [
    "GemmError", "gemm", "gemm_bf16", "gemm_f32", "gemm_naive_bf16",
    "gemm_naive_f32", "last_kernel", "library", "library_path",
]
