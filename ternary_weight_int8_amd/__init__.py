"""MI355X (gfx950) ternary x int8 GEMM: a C-ABI HIP library and its binding.

    ternary_gemm_s8(A, Wpacked)        C  = A x W        (W ternary, 2-bit packed)
    ternary_gemm_s8_dx(dC, Wpacked, K)  dX = dC x W^T
    ternary_gemm_s8_dw(A, dC)          dW = A^T x dC     (int8 x int8)

The library is loaded on first use and the calls raise if it is not built.
"""
from .binding import (  # noqa: F401
    TernaryGemmError,
    ternary_gemm_s8,
    ternary_gemm_s8_dw,
    ternary_gemm_s8_dx,
)
