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
ERR_NULL, ERR_DIM, ERR_PACK, ERR_BOUND, ERR_ALIAS, ERR_HIP, ERR_KIND, ERR_SCRATCH = -1, -2, -3, -4, -5, -6, -7, -8
STATIC_SCRATCH_BYTES = 8 << 20   # TGEMM_STATIC_SCRATCH_BYTES
OUT_F32, OUT_BF16 = 1, 2   # output kinds of the scaled calls
IN_F32, IN_BF16 = 1, 2     # input kinds of the quantizer calls

# entry points declared in include/ternary_gemm.h
EXPORTS = (
    "ternary_gemm_s8",
    "ternary_gemm_s8_dx",
    "ternary_gemm_s8_dw",
    "ternary_gemm_status_str",
    "ternary_gemm_plan",
    "ternary_gemm_plan_on",
    "ternary_gemm_machine",
    "ternary_gemm_tile_of",
    "ternary_gemm_s8_scaled",
    "ternary_gemm_s8_dx_scaled",
    "ternary_gemm_s8_dw_scaled",
    "ternary_pack_weights",
    "ternary_quantize_rows",
    "ternary_quantize_cols",
    "ternary_gemm_s8_dx_ws",
    "ternary_gemm_s8_dx_scaled_ws",
    "ternary_gemm_dx_workspace",
    "ternary_gemm_s8_dx_noalloc",
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
        ("xcds", ctypes.c_int32),
    ]


KERNEL_TILED, KERNEL_SPLIT, KERNEL_STREAM, KERNEL_SKINNY = 0, 2, 3, 4   # TgemmPlan.kernel


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
        L.ternary_gemm_plan_on.argtypes = [ctypes.c_int, i64, i64, i64, i64, ctypes.c_int32, ctypes.c_int32,
                                           ctypes.POINTER(TgemmPlan)]
        L.ternary_gemm_plan_on.restype = ctypes.c_int
        L.ternary_gemm_machine.argtypes = [ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int32)]
        L.ternary_gemm_machine.restype = ctypes.c_int
        L.ternary_gemm_tile_of.argtypes = [ctypes.POINTER(TgemmPlan), i64, i64,
                                           ctypes.POINTER(i64), ctypes.POINTER(i64)]
        L.ternary_gemm_tile_of.restype = ctypes.c_int
        f32, i32 = ctypes.c_float, ctypes.c_int
        for name in ("ternary_gemm_s8_scaled", "ternary_gemm_s8_dx_scaled"):
            f = getattr(L, name)
            f.argtypes = [p, p, p, f32, p, i32, i64, i64, i64, p]
            f.restype = ctypes.c_int
        L.ternary_gemm_s8_dw_scaled.argtypes = [p, p, p, p, p, i32, i64, i64, i64, p]
        L.ternary_gemm_s8_dw_scaled.restype = ctypes.c_int
        L.ternary_pack_weights.argtypes = [p, p, i64, i64, p]
        L.ternary_pack_weights.restype = ctypes.c_int
        for name in ("ternary_quantize_rows", "ternary_quantize_cols"):
            f = getattr(L, name)
            f.argtypes = [p, i32, p, p, i64, i64, p]
            f.restype = ctypes.c_int
        L.ternary_gemm_s8_dx_ws.argtypes = [p, p, p, i64, i64, i64, p, i64, p]
        L.ternary_gemm_s8_dx_ws.restype = ctypes.c_int
        L.ternary_gemm_s8_dx_scaled_ws.argtypes = [p, p, p, f32, p, i32, i64, i64, i64, p, i64, p]
        L.ternary_gemm_s8_dx_scaled_ws.restype = ctypes.c_int
        L.ternary_gemm_s8_dx_noalloc.argtypes = [p, p, p, i64, i64, i64, p]
        L.ternary_gemm_s8_dx_noalloc.restype = ctypes.c_int
        L.ternary_gemm_dx_workspace.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64)]
        L.ternary_gemm_dx_workspace.restype = ctypes.c_int
        _lib = L
    return _lib


def status_str(status: int) -> str:
    return lib().ternary_gemm_status_str(int(status)).decode()


def call_raw(name: str, p0, p1, p2, M: int, N: int, K: int, stream=None) -> int:
    """Call an entry point with raw addresses (ints or None); returns its status."""
    return getattr(lib(), name)(p0, p1, p2, M, N, K, stream)


def call_raw_scaled(name: str, p0, p1, s0, s1, out, kind: int, M: int, N: int, K: int, stream=None) -> int:
    """Call a scaled entry point with raw addresses; s1 is the weight scale
    (a float) for the forward and dX, the dC column scales' address for dW."""
    return getattr(lib(), name)(p0, p1, s0, s1, out, kind, M, N, K, stream)


def ternary_gemm_dx_workspace(M: int, N: int, K: int, align: int = 256) -> int:
    """Workspace bytes the dX calls with a workspace use (0: the one-pass kernels run)."""
    b = ctypes.c_int64()
    st = lib().ternary_gemm_dx_workspace(M, N, K, align, ctypes.byref(b))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_dx_workspace", st, status_str(st))
    return b.value


def machine():
    """(compute units, XCDs) of the current HIP device, as the calls plan for it."""
    cus, xcds = ctypes.c_int32(), ctypes.c_int32()
    st = lib().ternary_gemm_machine(ctypes.byref(cus), ctypes.byref(xcds))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_machine", st, status_str(st))
    return cus.value, xcds.value


def plan(op: str, M: int, N: int, K: int, align: int = 256, cus: int = None, xcds: int = None):
    """The launch plan of a call, for MI355X (256 CUs, 8 XCDs) unless cus and
    xcds name another machine."""
    pl = TgemmPlan()
    if cus is None and xcds is None:
        st = lib().ternary_gemm_plan(OPS[op], M, N, K, align, ctypes.byref(pl))
    else:
        st = lib().ternary_gemm_plan_on(OPS[op], M, N, K, align, cus, xcds, ctypes.byref(pl))
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


def _lowbit(addr: int) -> int:
    return addr & -addr if addr else 1 << 20


def _workspace(workspace, M, N, K, dC, Wpacked, stream):
    """The caller's workspace (a contiguous uint8 device tensor), or a new one
    of the size the library asks for; (address, bytes)."""
    torch = _torch()
    if workspace is None:
        align = min(_lowbit(dC.data_ptr()), _lowbit(Wpacked.data_ptr()))
        nbytes = ternary_gemm_dx_workspace(M, N, K, align)
        if nbytes == 0:
            return None, 0, None
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=dC.device)
        if stream is not None:
            workspace.record_stream(stream)   # freed here, in use on `stream`
    _check(workspace, torch.uint8, workspace.dim(), "workspace")
    if workspace.device != dC.device:
        raise ValueError(f"workspace must be on {dC.device}, got {workspace.device}")
    if workspace.numel() == 0:
        return None, 0, workspace
    return workspace.data_ptr(), workspace.numel(), workspace


def ternary_gemm_s8_dx_ws(dC, Wpacked, K, workspace=None, dX=None, stream=None):
    """ternary_gemm_s8_dx with a workspace (a contiguous uint8 device tensor of
    at least ternary_gemm_dx_workspace() bytes, empty for none; None: one of
    that size is allocated here)."""
    torch = _torch()
    _check(dC, torch.int8, 2, "dC")
    _check(Wpacked, torch.uint8, 2, "Wpacked")
    M, N = dC.shape
    if tuple(Wpacked.shape) != (N, K // 4) or K % 4:
        raise ValueError(f"Wpacked must be [N][K/4] = [{N}][{K // 4}], got {tuple(Wpacked.shape)}")
    dX = _output(dX, (M, K), torch.int32, dC.device, "dX")
    ws, nbytes, _keep = _workspace(workspace, M, N, K, dC, Wpacked, stream)
    st = lib().ternary_gemm_s8_dx_ws(dC.data_ptr(), Wpacked.data_ptr(), dX.data_ptr(), M, N, K, ws, nbytes,
                                     _stream(stream, dX.device))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_s8_dx_ws", st, status_str(st))
    return dX


def ternary_gemm_s8_dx_noalloc(dC, Wpacked, K, dX=None, stream=None):
    """ternary_gemm_s8_dx with the library's static device scratch in place of
    a workspace (the C call allocates nothing; dX is allocated here when not
    given)."""
    torch = _torch()
    _check(dC, torch.int8, 2, "dC")
    _check(Wpacked, torch.uint8, 2, "Wpacked")
    M, N = dC.shape
    if tuple(Wpacked.shape) != (N, K // 4) or K % 4:
        raise ValueError(f"Wpacked must be [N][K/4] = [{N}][{K // 4}], got {tuple(Wpacked.shape)}")
    dX = _output(dX, (M, K), torch.int32, dC.device, "dX")
    st = lib().ternary_gemm_s8_dx_noalloc(dC.data_ptr(), Wpacked.data_ptr(), dX.data_ptr(), M, N, K,
                                          _stream(stream, dX.device))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_s8_dx_noalloc", st, status_str(st))
    return dX


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


# ---------------------------------------------------------------------------
# scaled outputs: the integer product times per-row and per-column scales,
# stored as float32 or bfloat16
# ---------------------------------------------------------------------------

def _out_kind(dtype):
    torch = _torch()
    if dtype == torch.float32:
        return OUT_F32
    if dtype == torch.bfloat16:
        return OUT_BF16
    raise TypeError(f"out_dtype must be torch.float32 or torch.bfloat16, got {dtype}")


def _scales(t, n, what):
    torch = _torch()
    _check(t, torch.float32, 1, what)
    if t.shape[0] != n:
        raise ValueError(f"{what} must have {n} entries, got {t.shape[0]}")


def _output(out, shape, dtype, device, what):
    torch = _torch()
    if out is None:
        out = torch.empty(shape, dtype=dtype, device=device)
    _check(out, dtype, 2, what)
    if tuple(out.shape) != shape:
        raise ValueError(f"{what} must be {list(shape)}")
    return out


def ternary_gemm_s8_scaled(A, Wpacked, a_row_scale, w_scale, out_dtype=None, Y=None, stream=None):
    """Y [M][N] = (float(A x W) * a_row_scale[m]) * w_scale, float32 or bfloat16."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _check(A, torch.int8, 2, "A")
    _check(Wpacked, torch.uint8, 2, "Wpacked")
    M, K = A.shape
    N = Wpacked.shape[0]
    if Wpacked.shape[1] * 4 != K:
        raise ValueError(f"Wpacked must be [N][K/4] = [{N}][{K // 4}], got {tuple(Wpacked.shape)}")
    _scales(a_row_scale, M, "a_row_scale")
    Y = _output(Y, (M, N), out_dtype, A.device, "Y")
    st = lib().ternary_gemm_s8_scaled(A.data_ptr(), Wpacked.data_ptr(), a_row_scale.data_ptr(),
                                      float(w_scale), Y.data_ptr(), _out_kind(out_dtype), M, N, K,
                                      _stream(stream, Y.device))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_s8_scaled", st, status_str(st))
    return Y


def ternary_gemm_s8_dx_scaled(dC, Wpacked, K, dc_row_scale, w_scale, out_dtype=None, dX=None,
                              stream=None):
    """dX [M][K] = (float(dC x W^T) * dc_row_scale[m]) * w_scale, float32 or bfloat16."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _check(dC, torch.int8, 2, "dC")
    _check(Wpacked, torch.uint8, 2, "Wpacked")
    M, N = dC.shape
    if tuple(Wpacked.shape) != (N, K // 4) or K % 4:
        raise ValueError(f"Wpacked must be [N][K/4] = [{N}][{K // 4}], got {tuple(Wpacked.shape)}")
    _scales(dc_row_scale, M, "dc_row_scale")
    dX = _output(dX, (M, K), out_dtype, dC.device, "dX")
    st = lib().ternary_gemm_s8_dx_scaled(dC.data_ptr(), Wpacked.data_ptr(), dc_row_scale.data_ptr(),
                                         float(w_scale), dX.data_ptr(), _out_kind(out_dtype), M, N, K,
                                         _stream(stream, dX.device))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_s8_dx_scaled", st, status_str(st))
    return dX


def ternary_gemm_s8_dx_scaled_ws(dC, Wpacked, K, dc_row_scale, w_scale, out_dtype=None, workspace=None,
                                 dX=None, stream=None):
    """ternary_gemm_s8_dx_scaled with a workspace, as ternary_gemm_s8_dx_ws."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _check(dC, torch.int8, 2, "dC")
    _check(Wpacked, torch.uint8, 2, "Wpacked")
    M, N = dC.shape
    if tuple(Wpacked.shape) != (N, K // 4) or K % 4:
        raise ValueError(f"Wpacked must be [N][K/4] = [{N}][{K // 4}], got {tuple(Wpacked.shape)}")
    _scales(dc_row_scale, M, "dc_row_scale")
    dX = _output(dX, (M, K), out_dtype, dC.device, "dX")
    ws, nbytes, _keep = _workspace(workspace, M, N, K, dC, Wpacked, stream)
    st = lib().ternary_gemm_s8_dx_scaled_ws(dC.data_ptr(), Wpacked.data_ptr(), dc_row_scale.data_ptr(),
                                            float(w_scale), dX.data_ptr(), _out_kind(out_dtype), M, N, K,
                                            ws, nbytes, _stream(stream, dX.device))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_s8_dx_scaled_ws", st, status_str(st))
    return dX


def ternary_gemm_s8_dw_scaled(A, dC, a_col_scale, dc_col_scale, out_dtype=None, dW=None, stream=None):
    """dW [K][N] = (float(A^T x dC) * a_col_scale[k]) * dc_col_scale[n], float32 or bfloat16."""
    torch = _torch()
    out_dtype = out_dtype or torch.bfloat16
    _check(A, torch.int8, 2, "A")
    _check(dC, torch.int8, 2, "dC")
    M, K = A.shape
    if dC.shape[0] != M:
        raise ValueError("A and dC must have the same number of rows")
    N = dC.shape[1]
    _scales(a_col_scale, K, "a_col_scale")
    _scales(dc_col_scale, N, "dc_col_scale")
    dW = _output(dW, (K, N), out_dtype, A.device, "dW")
    st = lib().ternary_gemm_s8_dw_scaled(A.data_ptr(), dC.data_ptr(), a_col_scale.data_ptr(),
                                         dc_col_scale.data_ptr(), dW.data_ptr(), _out_kind(out_dtype),
                                         M, N, K, _stream(stream, dW.device))
    if st != OK:
        raise TernaryGemmError("ternary_gemm_s8_dw_scaled", st, status_str(st))
    return dW


# ---------------------------------------------------------------------------
# the steps before the product: packing the trainer's ternary weights, and
# per-row / per-column int8 quantization of activations
# ---------------------------------------------------------------------------

def ternary_pack_weights(Wt, Wpacked=None, stream=None):
    """Wpacked uint8 [N][K/4] from int8 weights Wt [N][K] (codes by sign)."""
    torch = _torch()
    _check(Wt, torch.int8, 2, "Wt")
    N, K = Wt.shape
    Wpacked = _output(Wpacked, (N, K // 4), torch.uint8, Wt.device, "Wpacked")
    st = lib().ternary_pack_weights(Wt.data_ptr(), Wpacked.data_ptr(), N, K, _stream(stream, Wt.device))
    if st != OK:
        raise TernaryGemmError("ternary_pack_weights", st, status_str(st))
    return Wpacked


def _quantize(name, X, Q, scale, n_scale, stream):
    torch = _torch()
    if not isinstance(X, torch.Tensor) or X.dtype not in (torch.float32, torch.bfloat16):
        raise TypeError("X must be a float32 or bfloat16 torch.Tensor")
    _check(X, X.dtype, 2, "X")
    R, C = X.shape
    Q = _output(Q, (R, C), torch.int8, X.device, "Q")
    n = R if n_scale == "rows" else C
    if scale is None:
        scale = torch.empty((n,), dtype=torch.float32, device=X.device)
    _scales(scale, n, "scale")
    kind = IN_F32 if X.dtype == torch.float32 else IN_BF16
    st = getattr(lib(), name)(X.data_ptr(), kind, Q.data_ptr(), scale.data_ptr(), R, C,
                              _stream(stream, X.device))
    if st != OK:
        raise TernaryGemmError(name, st, status_str(st))
    return Q, scale


def ternary_quantize_rows(X, Q=None, scale=None, stream=None):
    """(Q int8 [R][C], scale float32 [R]): per-row symmetric int8 quantization of X [R][C]."""
    return _quantize("ternary_quantize_rows", X, Q, scale, "rows", stream)


def ternary_quantize_cols(X, Q=None, scale=None, stream=None):
    """(Q int8 [R][C], scale float32 [C]): per-column symmetric int8 quantization of X [R][C]."""
    return _quantize("ternary_quantize_cols", X, Q, scale, "cols", stream)
