"""CPU oracle for the ternary x int8 GEMM -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its Python binding) never
does, and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C, int64 sums, threads split the
outer output index).  This module compiles it with gcc if ``liboracle.so`` is
absent and marshals numpy arrays into it.  Sources and the definitions
followed are listed at the top of ``oracle.c``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BUILD_CMD = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", _SRC, "-o", _LIB]


def build() -> str:
    """Compile liboracle.so (always; callers decide when)."""
    tmp = _LIB + ".tmp"
    cmd = BUILD_CMD[:-1] + [tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        lib.oracle_weight_of_code.argtypes = [ctypes.c_int]
        lib.oracle_weight_of_code.restype = ctypes.c_int
        for name in ("oracle_unpack", "oracle_pack", "oracle_decode"):
            getattr(lib, name).argtypes = [p, i64, i64, p]
            getattr(lib, name).restype = None
        for name in ("oracle_fwd", "oracle_dx", "oracle_dw"):
            getattr(lib, name).argtypes = [p, p, p, i64, i64, i64, ctypes.c_int]
            getattr(lib, name).restype = i64
        _lib = lib
    return _lib


def default_threads() -> int:
    """Threads for the oracle: the CPUs this process may run on, capped by
    OMP_NUM_THREADS when set (the share a job is given on a shared host)."""
    n = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {np.dtype(dtype)}, got {a.dtype}")
    return a


class OverflowInOracle(ArithmeticError):
    """An exact result left the int32 range."""


def weight_of_code(code: int) -> int:
    return int(_load().oracle_weight_of_code(int(code)))


def unpack(Wp: np.ndarray, K: int) -> np.ndarray:
    """Stored weights uint8 [N][K/4] -> codes uint8 [N][K]."""
    Wp = _c(Wp, np.uint8)
    N = Wp.shape[0]
    assert Wp.shape == (N, K // 4) and K % 4 == 0
    out = np.empty((N, K), dtype=np.uint8)
    _load().oracle_unpack(_ptr(Wp), N, K, _ptr(out))
    return out


def pack(codes: np.ndarray) -> np.ndarray:
    """Codes uint8 [N][K] (0..3) -> stored weights uint8 [N][K/4]."""
    codes = _c(codes, np.uint8)
    N, K = codes.shape
    assert K % 4 == 0
    out = np.empty((N, K // 4), dtype=np.uint8)
    _load().oracle_pack(_ptr(codes), N, K, _ptr(out))
    return out


def decode(Wp: np.ndarray, K: int) -> np.ndarray:
    """Stored weights uint8 [N][K/4] -> weights int8 [N][K] (w of (k, n) at [n][k])."""
    Wp = _c(Wp, np.uint8)
    N = Wp.shape[0]
    assert Wp.shape == (N, K // 4) and K % 4 == 0
    out = np.empty((N, K), dtype=np.int8)
    _load().oracle_decode(_ptr(Wp), N, K, _ptr(out))
    return out


def _run(name, X, Y, out, M, N, K, threads, allow_overflow):
    r = getattr(_load(), name)(_ptr(X), _ptr(Y), _ptr(out), M, N, K,
                               threads or default_threads())
    if r < 0:
        raise ValueError(f"{name}: bad arguments M={M} N={N} K={K}")
    if r and not allow_overflow:
        raise OverflowInOracle(f"{name}: {r} outputs outside int32")
    return out, int(r)


def fwd(A, Wp, threads=None, allow_overflow=False, return_overflows=False):
    """C int32 [M][N] = A int8 [M][K] x W, W stored as uint8 [N][K/4]."""
    A = _c(A, np.int8)
    Wp = _c(Wp, np.uint8)
    M, K = A.shape
    N = Wp.shape[0]
    assert Wp.shape == (N, K // 4) and K % 4 == 0
    C = np.empty((M, N), dtype=np.int32)
    C, r = _run("oracle_fwd", A, Wp, C, M, N, K, threads, allow_overflow)
    return (C, r) if return_overflows else C


def dx(dC, Wp, K, threads=None, allow_overflow=False, return_overflows=False):
    """dX int32 [M][K] = dC int8 [M][N] x W^T, same stored W as the forward."""
    dC = _c(dC, np.int8)
    Wp = _c(Wp, np.uint8)
    M, N = dC.shape
    assert Wp.shape == (N, K // 4) and K % 4 == 0
    dX = np.empty((M, K), dtype=np.int32)
    dX, r = _run("oracle_dx", dC, Wp, dX, M, N, K, threads, allow_overflow)
    return (dX, r) if return_overflows else dX


def dw(A, dC, threads=None, allow_overflow=False, return_overflows=False):
    """dW int32 [K][N] = A^T x dC, A int8 [M][K], dC int8 [M][N]."""
    A = _c(A, np.int8)
    dC = _c(dC, np.int8)
    M, K = A.shape
    assert dC.shape[0] == M
    N = dC.shape[1]
    dW = np.empty((K, N), dtype=np.int32)
    dW, r = _run("oracle_dw", A, dC, dW, M, N, K, threads, allow_overflow)
    return (dW, r) if return_overflows else dW
