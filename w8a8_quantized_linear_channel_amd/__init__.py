"""q8: an MI355X-native (gfx950) 8-bit quantized linear layer Y = X . W^T.

The compute lives in libq8.so (hand-written HIP kernels behind the C ABI of
include/q8.h).  This package only holds the ctypes binding (`ops`), the build
script (`build`) and the seeded synthetic input generators (`inputs`).
Importing the package does not load the library; the first call does, and
fails loudly if it is not built.
"""
from .ops import (  # noqa: F401
    q8_gemm_fp8,
    q8_gemm_int8,
    q8_linear,
    q8_linear_fp8,
    q8_linear_fp8_grouped,
    q8_linear_grouped,
    q8_linear_int8_decomp,
    q8_linear_noalloc,
    q8_linear_static,
    q8_linear_w8a16,
    q8_quantize_act,
    q8_quantize_act_static,
    q8_quantize_weight,
    q8_quantize_weight_grouped,
    q8_workspace_bytes,
)
