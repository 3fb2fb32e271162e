"""Python binding of libternary_gemm.so: argument marshalling only.

Every product runs in the library's HIP kernels.  There is no fallback: if the
library is missing or a call fails, these functions raise.  PyTorch supplies
device memory and the current stream; the library never allocates.
"""
from __future__ import annotations

import ctypes
import os

from .build import LIB

OK = 0
ERR_NULL, ERR_DIM, ERR_PACK, ERR_BOUND, ERR_ALIAS, ERR_HIP = -1, -2, -3, -4, -5, -6

# entry points declared in include/ternary_gemm.h
EXPORTS = (
    "ternary_gemm_s8",
    "ternary_gemm_s8_dx",
    "ternary_gemm_s8_dw",
    "ternary_gemm_status_str",
    "ternary_gemm_plan",
    "ternary_gemm_tile_of",
)

OPS = {"fwd": 0, "dx": 1, "dw": 2}


class TgemmPlan(ctypes.Structure):
    _fields_ = [
        ("out_rows", ctypes.c_int64), ("out_cols", ctypes.c_int64), ("contraction", ctypes.c_int64),
        ("tile_rows", ctypes.c_int32), ("tile_cols", ctypes.c_int32),
        ("tiles", ctypes.c_int64),
        ("workgroups", ctypes.c_int64),
        ("tiles_per_workgroup", ctypes.c_int64),
        ("band_cols", ctypes.c_int32),
        ("threads_per_workgroup", ctypes.c_int32), ("lds_bytes", ctypes.c_int32),
        ("fast_path", ctypes.c_int32), ("kernel", ctypes.c_int32),
    ]


KERNEL_TILED, KERNEL_SPLIT, KERNEL_STREAM = 0, 2, 3   # TgemmPlan.kernel


class TernaryGemmError(RuntimeError):
    def __init__(self, name, status, msg):
        super().__init__(f"{name}: status {status}: {msg}")
        self.status = status


_lib = None


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise RuntimeError(
                f"{LIB} is not built; run `python -c 'import __graft_entry__ as g; g.build()'`")
        L = ctypes.CDLL(LIB)
        p, i64 = ctypes.c_void_p, ctypes.c_int64
        for name in EXPORTS[:3]:
            f = getattr(L, name)
            f.argtypes = [p, p, p, i64, i64, i64, p]
            f.restype = ctypes.c_int
        L.ternary_gemm_status_str.argtypes = [ctypes.c_int]
        L.ternary_gemm_status_str.restype = ctypes.c_char_p
        L.ternary_gemm_plan.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.POINTER(TgemmPlan)]
        L.ternary_gemm_plan.restype = ctypes.c_int
        L.ternary_gemm_tile_of.argtypes = [ctypes.POINTER(TgemmPlan), i64, i64,
                                           ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.ternary_gemm_tile_of.restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().ternary_gemm_status_str(int(status)).decode()


def call_raw(name: str, p0, p1, p2, M: int, N: int, K: int, stream=None) -> int:
    """Call an entry point with raw addresses (ints or None); returns its status."""
    return getattr(lib(), name)(p0, p1, p2, M, N, K, stream)


def plan(op: str, M: int, N: int, K: int, align: int = 256):
    pl = TgemmPlan()
    st = lib().ternary_gemm_plan(OPS[op], M, N, K, align, ctypes.byref(pl))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_plan", st, status_str(st))
    return pl


def tile_of(pl: TgemmPlan, workgroup: int, iteration: int = 0):
    """(row0, col0) of the tile a workgroup computes in one iteration, or None if none."""
    r, c = ctypes.c_int64(), ctypes.c_int64()
    st = lib().ternary_gemm_tile_of(ctypes.byref(pl), workgroup, iteration, ctypes.byref(r),
                                    ctypes.byref(c))
    if st == ERR_DIM and 0 <= workgroup < pl.workgroups and 0 <= iteration < pl.tiles_per_workgroup:
        return None
    if st != OK:
        raise TernaryGemmError("ternary_gemm_tile_of", st, status_str(st))
    return r.value, c.value


# ---------------------------------------------------------------------------
# torch-tensor wrappers (same names as the C entry points)
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _check(t, dtype, ndim, what):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{what} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{what} must be {ndim}-D, got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{what} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{what} must be contiguous")


def _stream(stream, device):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream(device)
    return ctypes.c_void_p(s.cuda_stream)


def _invoke(name, a, b, out, M, N, K, stream):
    st = getattr(lib(), name)(a.data_ptr(), b.data_ptr(), out.data_ptr(), M, N, K,
                              _stream(stream, out.device))
    if st != OK:
        raise TernaryGemmError(name, st, status_str(st))
    return out


def ternary_gemm_s8(A, Wpacked, C=None, stream=None):
    """C int32 [M][N] = A int8 [M][K] x W, W stored as uint8 [N][K/4]."""
    torch = _torch()
    _check(A, torch.int8, 2, "A")
    _check(Wpacked, torch.uint8, 2, "Wpacked")
    M, K = A.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 4 != K:
        raise ValueError(f"Wpacked must be [N][K/4] = [{N}][{K // 4}], got {tuple(Wpacked.shape)}")
    if C is None:
        C = torch.empty((M, N), dtype=torch.int32, device=A.device)
    _check(C, torch.int32, 2, "C")
    if tuple(C.shape) != (M, N):
        raise ValueError(f"C must be [{M}][{N}]")
    return _invoke("ternary_gemm_s8", A, Wpacked, C, M, N, K, stream)


def ternary_gemm_s8_dx(dC, Wpacked, K, dX=None, stream=None):
    """dX int32 [M][K] = dC int8 [M][N] x W^T, same stored W as the forward."""
    torch = _torch()
    _check(dC, torch.int8, 2, "dC")
    _check(Wpacked, torch.uint8, 2, "Wpacked")
    M, N = dC.shape
    if tuple(Wpacked.shape) != (N, K // 4) or K % 4:
        raise ValueError(f"Wpacked must be [N][K/4] = [{N}][{K // 4}], got {tuple(Wpacked.shape)}")
    if dX is None:
        dX = torch.empty((M, K), dtype=torch.int32, device=dC.device)
    _check(dX, torch.int32, 2, "dX")
    if tuple(dX.shape) != (M, K):
        raise ValueError(f"dX must be [{M}][{K}]")
    return _invoke("ternary_gemm_s8_dx", dC, Wpacked, dX, M, N, K, stream)


def ternary_gemm_s8_dw(A, dC, dW=None, stream=None):
    """dW int32 [K][N] = A^T x dC, A int8 [M][K], dC int8 [M][N]."""
    torch = _torch()
    _check(A, torch.int8, 2, "A")
    _check(dC, torch.int8, 2, "dC")
    M, K = A.shape
    if dC.shape[0] != M:
        raise ValueError("A and dC must have the same number of rows")
    N = dC.shape[1]
    if dW is None:
        dW = torch.empty((K, N), dtype=torch.int32, device=A.device)
    _check(dW, torch.int32, 2, "dW")
    if tuple(dW.shape) != (K, N):
        raise ValueError(f"dW must be [{K}][{N}]")
    return _invoke("ternary_gemm_s8_dw", A, dC, dW, M, N, K, stream)
