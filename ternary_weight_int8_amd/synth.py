"""Seeded synthetic inputs for the ternary x int8 GEMM and its backward-style variants.

This module only draws random bytes. It holds none of the GEMM's arithmetic
(no weight decode, no products, no sums) so that the HIP path and the CPU oracle
can both consume exactly the same input bytes without sharing any of the method.

Generator: counter-based SplitMix64 (Steele, Lea and Flood, "Fast splittable
pseudorandom number generators", OOPSLA 2014; the output mixer is the variant
with the constants published in Vigna's public splitmix64.c):

    gamma      = 0x9E3779B97F4A7C15
    mix64(z)   = z ^= z >> 30; z *= 0xBF58476D1CE4E5B9;
                 z ^= z >> 27; z *= 0x94D049BB133111EB; z ^= z >> 31
    base(s, t) = mix64(s ^ (t * gamma))
    u(s, t, i) = mix64(base(s, t) + (i + 1) * gamma)          (all mod 2**64)

i.e. value i of stream t is the (i+1)-th output of a sequential SplitMix64
whose state starts at base(s, t).  Streams: 0 = A (activations), 1 = weight
codes, 2 = dC (incoming gradient).  The index i is the element's storage index
(m*K + k for A, n*K + k for the code of weight (k, n), m*N + n for dC).

Value maps (u is the 64-bit draw):
    int8 uniform over [-128, 127]   : top byte of u, read as two's complement
    code uniform over {0, 1, 2, 3}  : u >> 62
    code uniform over {0, 1, 2}     : ((u >> 32) * 3) >> 32   (multiply-shift)

Stored weights: W[K, N] is kept as 2-bit codes, 4 per byte, N-major: the code
of (k, n) sits in byte n*(K/4) + k//4 at bits 2*(k%4) .. 2*(k%4)+1 (the first
code of a byte in its least significant bits).  The t27 pages give the 4-per-
byte packing and the N-major code index (t27 pull request #10425 "t27c PTX
backend: ternary x int8 GEMM kernel emitted by a .t27 spec", section "What
this adds"; t27 pull request #10855 "hslm_bwd_ptx -- HSLM backward dX and dW",
PR body, index layout code[j*K + i]); the order of codes inside a byte is not
stated there, and least-significant-first is the reading taken.

The workload shapes below are the pages' own: the ragged 300x272x96 and tiny
1x16x16 correctness shapes and the 16384x3456x1280 "500m" shape (#10425,
results comment, "Bit-exact" and "Throughput" tables), and the HSLM backward
pair at 1782 rows (#10855, commit message and "Measured").
"""
from __future__ import annotations

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

STREAM_A = 0
STREAM_CODES = 1
STREAM_DC = 2
STREAM_ROW_SCALE = 3
STREAM_COL_SCALE = 4
STREAM_X = 5            # floating-point activations (quantizer input)
STREAM_TERNARY = 6      # the trainer's ternary weights (packer input)

# elements generated per numpy pass; bounds the temporaries to a few hundred MB
_CHUNK = 1 << 24


def _mix64(z: np.ndarray) -> np.ndarray:
    z = z ^ (z >> np.uint64(30))
    z = z * _M1
    z = z ^ (z >> np.uint64(27))
    z = z * _M2
    return z ^ (z >> np.uint64(31))


def stream_base(seed: int, stream: int) -> int:
    """Starting state of stream `stream` under seed `seed`."""
    with np.errstate(over="ignore"):
        s = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) ^ (np.uint64(stream) * GAMMA)
        return int(_mix64(np.array([s], dtype=np.uint64))[0])


def splitmix64(seed: int, stream: int, count: int, offset: int = 0) -> np.ndarray:
    """u(seed, stream, i) for i in [offset, offset + count), as uint64."""
    base = np.uint64(stream_base(seed, stream))
    out = np.empty(count, dtype=np.uint64)
    with np.errstate(over="ignore"):
        for lo in range(0, count, _CHUNK):
            hi = min(count, lo + _CHUNK)
            idx = np.arange(offset + lo + 1, offset + hi + 1, dtype=np.uint64)
            out[lo:hi] = _mix64(base + idx * GAMMA)
    return out


def _map_chunks(seed, stream, count, fn, dtype):
    out = np.empty(count, dtype=dtype)
    for lo in range(0, count, _CHUNK):
        hi = min(count, lo + _CHUNK)
        out[lo:hi] = fn(splitmix64(seed, stream, hi - lo, offset=lo))
    return out


def _u_to_int8(u: np.ndarray) -> np.ndarray:
    return (u >> np.uint64(56)).astype(np.uint8).view(np.int8)


def _u_to_code4(u: np.ndarray) -> np.ndarray:
    return (u >> np.uint64(62)).astype(np.uint8)


def _u_to_code3(u: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return (((u >> np.uint64(32)) * np.uint64(3)) >> np.uint64(32)).astype(np.uint8)


def uniform_int8(seed: int, stream: int, rows: int, cols: int) -> np.ndarray:
    """int8 [rows][cols], uniform over [-128, 127]."""
    return _map_chunks(seed, stream, rows * cols, _u_to_int8, np.int8).reshape(rows, cols)


def random_codes(seed: int, N: int, K: int, alphabet: int) -> np.ndarray:
    """uint8 [N][K] of 2-bit codes, uniform over {0..alphabet-1} (alphabet 3 or 4)."""
    if alphabet == 4:
        fn = _u_to_code4
    elif alphabet == 3:
        fn = _u_to_code3
    else:
        raise ValueError("alphabet must be 3 or 4")
    return _map_chunks(seed, STREAM_CODES, N * K, fn, np.uint8).reshape(N, K)


def store_codes(codes: np.ndarray) -> np.ndarray:
    """Place uint8 codes [N][K] (values 0..3) into the stored form uint8 [N][K/4].

    Pure bit placement: code (k, n) goes to bits 2*(k%4) of byte n*(K/4)+k//4.
    """
    N, K = codes.shape
    if K % 4:
        raise ValueError("K must be a multiple of 4 for the 4-codes-per-byte form")
    c = codes.reshape(N, K // 4, 4).astype(np.uint8) & np.uint8(3)
    return (c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)).astype(np.uint8)


def stored_weights(seed: int, N: int, K: int, alphabet: int) -> np.ndarray:
    """Random stored weights uint8 [N][K/4], codes uniform over {0..alphabet-1}."""
    return store_codes(random_codes(seed, N, K, alphabet))


# --------------------------------------------------------------------------
# The workloads.  Each is a dict of shapes plus the recipe of its inputs.
# --------------------------------------------------------------------------

CONFIGS = {
    # 1 x 16 x 16, codes over {0,1,2,3} (code 3 exercised)
    "tiny": dict(op="fwd", M=1, N=16, K=16, alphabet=4),
    # 300 x 272 x 96, no dimension a tile multiple: every edge guard
    "ragged": dict(op="fwd", M=300, N=272, K=96, alphabet=4),
    # 16384 x 3456 x 1280, the "500m" throughput shape, codes over {0,1,2}
    "large": dict(op="fwd", M=16384, N=3456, K=1280, alphabet=3),
    # 2048 x 2048 x 65536 with structured halves (see extreme_inputs)
    "extreme": dict(op="fwd", M=2048, N=2048, K=65536, alphabet=None),
    # HSLM backward pair at 1782 rows: dX with the same stored W, and dW
    "backward": dict(op="bwd", M=1782, N=3456, K=1280, alphabet=3),
}


def fwd_inputs(seed: int, M: int, N: int, K: int, alphabet: int):
    """(A int8 [M][K], Wp uint8 [N][K/4]) for the forward product."""
    return uniform_int8(seed, STREAM_A, M, K), stored_weights(seed, N, K, alphabet)


def dx_inputs(seed: int, M: int, N: int, K: int, alphabet: int):
    """(dC int8 [M][N], Wp uint8 [N][K/4]) for dX = dC x W^T."""
    return uniform_int8(seed, STREAM_DC, M, N), stored_weights(seed, N, K, alphabet)


def dw_inputs(seed: int, M: int, N: int, K: int):
    """(A int8 [M][K], dC int8 [M][N]) for dW = A^T x dC."""
    return uniform_int8(seed, STREAM_A, M, K), uniform_int8(seed, STREAM_DC, M, N)


def extreme_inputs(seed: int, M: int, N: int, K: int):
    """Structured stress inputs at the int32 accumulation bound.

    Rows m < M/2 of A are all -128; rows m >= M/2 are uniform int8 (drawn at
    their storage indices, so the rows do not depend on M's lower half).
    Columns n < N/2 of W hold code 1 (+1) everywhere, the others code 2 (-1):
    stored bytes 0x55 and 0xAA.
    """
    A = np.full((M, K), -128, dtype=np.int8)
    h = M // 2
    if M - h:
        u = splitmix64(seed, STREAM_A, (M - h) * K, offset=h * K)
        A[h:] = _u_to_int8(u).reshape(M - h, K)
    Wp = np.empty((N, K // 4), dtype=np.uint8)
    Wp[: N // 2] = 0x55
    Wp[N // 2:] = 0xAA
    return A, Wp


def positive_scales(seed: int, stream: int, n: int, lo: float = 2.0 ** -10, hi: float = 2.0 ** -3) -> np.ndarray:
    """float32 [n], log-uniform over [lo, hi): per-row or per-column scales for
    the scaled outputs (the range of absmax / 127 of int8-quantized values)."""
    u = splitmix64(seed, stream, n)
    t = (u >> np.uint64(11)).astype(np.float64) / float(1 << 53)
    return (lo * (hi / lo) ** t).astype(np.float32)


# the weight scale of the scaled forward and dX calls in tests and benchmarks
W_SCALE = 0.0371


def float_inputs(seed: int, stream: int, rows: int, cols: int, kind: str) -> np.ndarray:
    """Finite floating-point inputs for the quantizer, drawn as bit patterns:
    "f32" gives float32 [rows][cols], "bf16" the bfloat16 bit patterns as
    uint16 [rows][cols].  Each element takes a random sign, a binary exponent
    uniform over -8 .. 3 and a random mantissa; about one element in 256 is
    +0 or -0.  (Bits only: no rounding takes place here.)"""
    u = splitmix64(seed, stream, rows * cols)
    sign = (u >> np.uint64(63)).astype(np.uint32)
    e = ((((u >> np.uint64(32)) & np.uint64(0xFFFFFFFF)) * np.uint64(12)) >> np.uint64(32)).astype(np.uint32)
    e = e + np.uint32(127 - 8)                     # biased exponent, 2^-8 .. 2^3
    zero = (u & np.uint64(0xFF)) == 0
    if kind == "f32":
        mant = ((u >> np.uint64(8)) & np.uint64((1 << 23) - 1)).astype(np.uint32)
        bits = (sign << np.uint32(31)) | (e << np.uint32(23)) | mant
        bits = np.where(zero, sign << np.uint32(31), bits).astype(np.uint32)
        return bits.view(np.float32).reshape(rows, cols)
    if kind == "bf16":
        mant = ((u >> np.uint64(8)) & np.uint64(0x7F)).astype(np.uint32)
        bits = (sign << np.uint32(15)) | (e << np.uint32(7)) | mant
        bits = np.where(zero, sign << np.uint32(15), bits)
        return bits.astype(np.uint16).reshape(rows, cols)
    raise ValueError(kind)


def ternary_int8(seed: int, N: int, K: int) -> np.ndarray:
    """The trainer's ternary weights int8 [N][K] (row n: the K weights of
    output column n, the layout of a linear layer's weight), each uniform
    over {-1, 0, +1}: a uniform draw over {0, 1, 2} minus one."""
    u = splitmix64(seed, STREAM_TERNARY, N * K)
    return (_u_to_code3(u).astype(np.int16) - 1).astype(np.int8).reshape(N, K)
