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
_DEFAULT_LIB = os.path.join(_HERE, "liboracle.so")
# TERNARY_ORACLE_LIB names another build of oracle.c to load instead (the
# sanitizer test's; it is never built here)
_LIB = os.environ.get("TERNARY_ORACLE_LIB") or _DEFAULT_LIB

BUILD_CMD = ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-pthread", _SRC, "-o", _DEFAULT_LIB]
SANITIZE_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                  "-fno-sanitize-recover=all"]


def build() -> str:
    """Compile liboracle.so (always; callers decide when)."""
    tmp = _DEFAULT_LIB + ".tmp"
    cmd = BUILD_CMD[:-1] + [tmp]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _DEFAULT_LIB)
    return _DEFAULT_LIB


def build_sanitized(path: str) -> str:
    """Compile oracle.c with AddressSanitizer and UndefinedBehaviorSanitizer
    (host code only) into `path`."""
    subprocess.run(["gcc", *SANITIZE_FLAGS, "-std=c99", "-fPIC", "-shared", "-pthread", _SRC, "-o", path],
                   check=True)
    return path


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            if _LIB != _DEFAULT_LIB:
                raise RuntimeError(f"TERNARY_ORACLE_LIB={_LIB} does not exist")
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


# ---------------------------------------------------------------------------
# Scaled outputs: the dequantization that follows the integer product.  The
# pages leave the scales to the host (activations per row for dX, X and dY
# per column for dW [P10855 PR body]); the reading taken is
#     y = (float32(acc) * row_scale[row]) * col_scale[col]
# in IEEE single precision, each step rounded to nearest even, in that order,
# then optionally rounded to the nearest bfloat16, ties to even.
# ---------------------------------------------------------------------------

def bf16_value(bits) -> np.ndarray:
    """float64 value of bfloat16 bit patterns (uint16), finite or not: an
    all-ones exponent is taken as the next power of two past the largest
    finite value (2^128), the value that rounding to bf16 overflows to."""
    b = np.asarray(bits, dtype=np.uint32)
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = ((b >> 7) & 0xFF).astype(np.int64)
    m = (b & 0x7F).astype(np.float64)
    mag = np.where(e == 0, np.ldexp(m, -133), np.ldexp(128.0 + m, (e - 134).astype(np.int64)))
    return sign * mag


def bf16_nearest_even(x) -> np.ndarray:
    """bfloat16 bit patterns (uint16) of float32 values: the nearest bf16,
    ties to the one with an even last mantissa bit; +-inf stay inf, values at
    or past the midpoint above the largest finite bf16 become inf, and a NaN
    becomes a quiet NaN with the same sign and top payload bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lo = (u >> 16) & 0xFFFF                        # toward zero
    hi = lo + 1                                    # away from zero (same sign)
    xv = x.astype(np.float64)
    d_lo = np.abs(xv - bf16_value(lo))
    d_hi = np.abs(bf16_value(hi) - xv)
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((lo & 1) == 1))
    out = np.where(pick_hi, hi, lo)
    out = np.where(np.isinf(x), lo, out)
    out = np.where(np.isnan(x), lo | 0x40, out)
    return out.astype(np.uint16)


def scale_output(acc, row_scale, col_scale, out: str) -> np.ndarray:
    """Scaled output of an integer result acc [R][C]: row_scale float32 [R],
    col_scale float32 [C] or one float32 for every column; out "f32" gives
    float32 [R][C], "bf16" the bfloat16 bit patterns as uint16 [R][C]."""
    acc = np.asarray(acc)
    if acc.dtype != np.int32:
        raise TypeError("acc must be int32")
    rs = np.asarray(row_scale, dtype=np.float32)
    assert rs.shape == (acc.shape[0],)
    y = acc.astype(np.float32) * rs[:, None]
    cs = np.asarray(col_scale, dtype=np.float32)
    y = y * (cs[None, :] if cs.ndim else cs)
    assert y.dtype == np.float32
    if out == "f32":
        return y
    if out == "bf16":
        return bf16_nearest_even(y)
    raise ValueError(f"out must be 'f32' or 'bf16', got {out!r}")


# ---------------------------------------------------------------------------
# The steps before the product.
#
# Packing the trainer's ternary weights: the stored format is the pages'
# (2-bit codes, four per byte along K, one row of K/4 bytes per output column
# n; codes 0, 1, 2 stand for 0, +1, -1 [P10425 "What this adds"; P10855 PR
# body]); the pages leave wiring the trainer to it for later.  The reading
# taken: the input is int8 [N][K] (row n holds output column n's weights, as a
# linear layer stores them), and a weight's code is chosen by its sign:
# 1 for w > 0, 2 for w < 0, 0 for w == 0, so {-1, 0, +1} map to their codes
# and code 3 is never produced.
#
# Quantizing activations to int8: the pages give only where the scales go
# (per row for the forward's A and dX's dC; per column of X and dY for dW
# [P10855 PR body]).  The reading taken is the plain symmetric absmax rule,
# in IEEE single precision with nearest-even rounding at each step:
#     s = max|x| / 127          over the row (or column)
#     q = clamp(rint(x / s), -127, 127)      (q = 0 where s == 0)
# so that q * s approximates x and a scaled output is (acc * s_row) * s_col.
# ---------------------------------------------------------------------------

def ternary_codes(Wt) -> np.ndarray:
    """Codes uint8 [N][K] of int8 weights [N][K]: 1 if w > 0, 2 if w < 0, else 0."""
    w = np.asarray(Wt, dtype=np.int8)
    return np.where(w > 0, 1, np.where(w < 0, 2, 0)).astype(np.uint8)


def pack_weights(Wt) -> np.ndarray:
    """Stored weights uint8 [N][K/4] of int8 weights [N][K] (codes by sign)."""
    return pack(ternary_codes(Wt))


def as_float32(X, kind: str) -> np.ndarray:
    """Values of the quantizer's input as float32 ("f32": float32 array;
    "bf16": bfloat16 bit patterns, uint16, widened exactly)."""
    if kind == "f32":
        return np.ascontiguousarray(X, dtype=np.float32)
    if kind == "bf16":
        b = np.ascontiguousarray(X, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
        return b.view(np.float32)
    raise ValueError(kind)


def quantize(X, kind: str, axis: str):
    """Symmetric int8 quantization of X [R][C]: axis "rows" gives one scale per
    row (scale float32 [R]), "cols" one per column (scale float32 [C]).
    Returns (q int8 [R][C], scale)."""
    x = as_float32(X, kind)
    ax = {"rows": 1, "cols": 0}[axis]
    amax = np.abs(x).max(axis=ax) if x.size else np.zeros(x.shape[1 - ax], np.float32)
    s = (amax.astype(np.float32) / np.float32(127)).astype(np.float32)
    sb = s[:, None] if axis == "rows" else s[None, :]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(x / sb)
    q = np.where(sb > 0, np.clip(r, -127, 127), 0).astype(np.int8)
    return q, s
