"""GPU parity: the HIP library against the CPU oracle, element by element.

All products are exact integer results, so the bar is bit-exact equality
(mismatch count 0) on every seeded input.  The oracle computes every element
of every case here, the 16384 x 3456 x 1280 forward included; the structured
2048 x 2048 x 65536 stress case is checked in full against its closed form and
on sampled rows against the oracle.
"""
import sys

import numpy as np
import pytest

import oracle
from ternary_weight_int8_amd import binding as B
from ternary_weight_int8_amd import synth
from shapes import (DW_SHAPES, DX_SHAPES, DX_STREAM_SHAPES, FWD_SHAPES, SKINNY_DX_SHAPES,
                    SKINNY_SHAPES, STREAM_SHAPES)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def assert_exact(got, want, what):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if len(bad):
        first = [(tuple(int(v) for v in ix), int(got[tuple(ix)]), int(want[tuple(ix)])) for ix in bad[:8]]
        pytest.fail(f"{what}: {len(bad)} mismatches of {got.size}; first (index, gpu, oracle): {first}")


def gpu_fwd(A, Wp):
    return host(B.ternary_gemm_s8(dev(A), dev(Wp)))


def gpu_dx(dC, Wp, K):
    return host(B.ternary_gemm_s8_dx(dev(dC), dev(Wp), K))


def gpu_dw(A, dC):
    return host(B.ternary_gemm_s8_dw(dev(A), dev(dC)))


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed", range(16))
def test_tiny(seed):
    c = synth.CONFIGS["tiny"]
    say(f"tiny seed={seed}")
    A, Wp = synth.fwd_inputs(seed, c["M"], c["N"], c["K"], c["alphabet"])
    assert_exact(gpu_fwd(A, Wp), oracle.fwd(A, Wp), f"tiny seed {seed}")


@pytest.mark.parametrize("seed", range(16))
def test_ragged(seed):
    c = synth.CONFIGS["ragged"]
    say(f"ragged seed={seed}")
    A, Wp = synth.fwd_inputs(seed, c["M"], c["N"], c["K"], c["alphabet"])
    assert_exact(gpu_fwd(A, Wp), oracle.fwd(A, Wp), f"ragged seed {seed}")


@pytest.fixture(scope="module")
def large_inputs():
    c = synth.CONFIGS["large"]
    return synth.fwd_inputs(1, c["M"], c["N"], c["K"], c["alphabet"])


def test_large_full(large_inputs):
    say("large 16384x3456x1280 seed=1, every element")
    A, Wp = large_inputs
    assert_exact(gpu_fwd(A, Wp), oracle.fwd(A, Wp), "large seed 1")


def test_large_backward_full(large_inputs):
    # dX and dW at the timed shape, on the same inputs the benchmark draws
    c = synth.CONFIGS["large"]
    M, N, K = c["M"], c["N"], c["K"]
    A, Wp = large_inputs
    dC = synth.uniform_int8(1, synth.STREAM_DC, M, N)
    say("large dX 16384x3456x1280 seed=1, every element")
    assert_exact(gpu_dx(dC, Wp, K), oracle.dx(dC, Wp, K), "large dX")
    say("large dW 16384x3456x1280 seed=1, every element")
    assert_exact(gpu_dw(A, dC), oracle.dw(A, dC), "large dW")


@pytest.mark.parametrize("seed", [2, 3])
def test_large_other_seeds(seed):
    # every element against the oracle, and the whole tensor against the row-
    # and column-sum identities, which hold for the exact product at any size
    c = synth.CONFIGS["large"]
    M, N, K = c["M"], c["N"], c["K"]
    say(f"large seed={seed}, every element + sum identities")
    A, Wp = synth.fwd_inputs(seed, M, N, K, c["alphabet"])
    C = gpu_fwd(A, Wp)
    assert_exact(C, oracle.fwd(A, Wp), f"large seed {seed}")
    w = oracle.decode(Wp, K).astype(np.int64)              # [N][K]
    A64 = A.astype(np.int64)
    np.testing.assert_array_equal(C.astype(np.int64).sum(axis=1), A64 @ w.sum(axis=0))
    np.testing.assert_array_equal(C.astype(np.int64).sum(axis=0), w @ A64.sum(axis=0))


def test_extreme():
    c = synth.CONFIGS["extreme"]
    M, N, K = c["M"], c["N"], c["K"]
    say("extreme 2048x2048x65536 closed form + sampled rows")
    A, Wp = synth.extreme_inputs(1, M, N, K)
    C = gpu_fwd(A, Wp)
    sign = np.where(np.arange(N) < N // 2, 1, -1).astype(np.int64)
    want = A.astype(np.int64).sum(axis=1)[:, None] * sign[None, :]
    assert_exact(C.astype(np.int64), want, "extreme closed form")
    assert (C[: M // 2, : N // 2] == -128 * K).all() and (C[: M // 2, N // 2:] == 128 * K).all()
    rows = np.array([0, 1, M // 2 - 1, M // 2, M // 2 + 1, M - 2, M - 1])
    assert_exact(C[rows], oracle.fwd(A[rows], Wp), "extreme rows vs oracle")


@pytest.mark.parametrize("seed", [1, 2])
def test_backward_pair(seed):
    c = synth.CONFIGS["backward"]
    M, N, K = c["M"], c["N"], c["K"]
    say(f"backward dX seed={seed}")
    dC, Wp = synth.dx_inputs(seed, M, N, K, c["alphabet"])
    assert_exact(gpu_dx(dC, Wp, K), oracle.dx(dC, Wp, K), f"dX seed {seed}")
    say(f"backward dW seed={seed}")
    A, dC2 = synth.dw_inputs(seed, M, N, K)
    assert_exact(gpu_dw(A, dC2), oracle.dw(A, dC2), f"dW seed {seed}")


# ---------------------------------------------------------------------------
# every tile shape x load path, with ragged edges in all three dimensions
# ---------------------------------------------------------------------------

def tile_of(op, M, N, K):
    pl = B.plan(op, M, N, K)
    return pl.tile_rows, pl.tile_cols, pl.fast_path


@pytest.mark.parametrize("M,N,K", FWD_SHAPES)
def test_fwd_shapes(M, N, K):
    say(f"fwd {M}x{N}x{K} plan={tile_of('fwd', M, N, K)}")
    A, Wp = synth.fwd_inputs(M * 7 + K, M, N, K, 4)
    assert_exact(gpu_fwd(A, Wp), oracle.fwd(A, Wp), f"fwd {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", STREAM_SHAPES)
def test_fwd_stream_shapes(M, N, K):
    say(f"fwd stream {M}x{N}x{K} plan={tile_of('fwd', M, N, K)}")
    A, Wp = synth.fwd_inputs(M * 11 + K, M, N, K, 4)
    assert_exact(gpu_fwd(A, Wp), oracle.fwd(A, Wp), f"fwd stream {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", SKINNY_SHAPES)
def test_fwd_skinny_shapes(M, N, K):
    say(f"fwd skinny {M}x{N}x{K} plan={tile_of('fwd', M, N, K)}")
    assert B.plan("fwd", M, N, K).kernel == B.KERNEL_SKINNY
    A, Wp = synth.fwd_inputs(M * 13 + N + K, M, N, K, 4)
    assert_exact(gpu_fwd(A, Wp), oracle.fwd(A, Wp), f"fwd skinny {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", SKINNY_DX_SHAPES)
def test_dx_skinny_shapes(M, N, K):
    say(f"dx skinny {M}x{N}x{K} plan={tile_of('dx', M, N, K)}")
    assert B.plan("dx", M, N, K).kernel == B.KERNEL_SKINNY
    dC, Wp = synth.dx_inputs(M * 17 + N + K, M, N, K, 4)
    assert_exact(gpu_dx(dC, Wp, K), oracle.dx(dC, Wp, K), f"dx skinny {M}x{N}x{K}")


def test_skinny_extreme():
    # the int32 extremes through the skinny kernel: A row 0 all -128, row 1
    # uniform; codes +1 in columns < 16, -1 in the rest; K = 16777152, the
    # longest whole number of 64-steps inside the exact-int32 bound
    M, N, K = 2, 32, 16777152
    say(f"fwd skinny extreme {M}x{N}x{K}")
    assert B.plan("fwd", M, N, K).kernel == B.KERNEL_SKINNY
    A, Wp = synth.extreme_inputs(1, M, N, K)
    C = gpu_fwd(A, Wp)
    assert (C[0, :16] == -128 * K).all() and (C[0, 16:] == 128 * K).all()
    assert -128 * K == -2147475456
    assert_exact(C, oracle.fwd(A, Wp), "skinny extreme vs oracle")


@pytest.mark.parametrize("M,N,K", DX_STREAM_SHAPES)
def test_dx_stream_shapes(M, N, K):
    say(f"dx stream {M}x{N}x{K} plan={tile_of('dx', M, N, K)}")
    dC, Wp = synth.dx_inputs(M * 13 + N, M, N, K, 4)
    assert_exact(gpu_dx(dC, Wp, K), oracle.dx(dC, Wp, K), f"dx stream {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", DX_SHAPES)
def test_dx_shapes(M, N, K):
    say(f"dx {M}x{N}x{K} plan={tile_of('dx', M, N, K)}")
    dC, Wp = synth.dx_inputs(M * 5 + N, M, N, K, 4)
    assert_exact(gpu_dx(dC, Wp, K), oracle.dx(dC, Wp, K), f"dx {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", DW_SHAPES)
def test_dw_shapes(M, N, K):
    say(f"dw {M}x{N}x{K} plan={tile_of('dw', M, N, K)}")
    A, dC = synth.dw_inputs(M * 3 + K, M, N, K)
    assert_exact(gpu_dw(A, dC), oracle.dw(A, dC), f"dw {M}x{N}x{K}")


# ---------------------------------------------------------------------------
# alignment, coverage, determinism
# ---------------------------------------------------------------------------

def offset_view(x_np, offset):
    """Device copy of x starting `offset` bytes into a fresh buffer (misaligned base)."""
    flat = np.ascontiguousarray(x_np).reshape(-1).view(np.uint8)
    buf = torch.zeros(flat.size + 64, dtype=torch.uint8, device=DEV)
    buf[offset:offset + flat.size] = torch.from_numpy(flat).to(DEV)
    v = buf[offset:offset + flat.size]
    return v.view(torch.int8 if x_np.dtype == np.int8 else torch.uint8).view(*x_np.shape)


@pytest.mark.parametrize("offset", [1, 2, 4, 8])
def test_misaligned_bases(offset):
    M, N, K = 300, 272, 96
    say(f"misaligned by {offset}")
    A, Wp = synth.fwd_inputs(offset, M, N, K, 4)
    Ad, Wd = offset_view(A, offset), offset_view(Wp, offset)
    assert Ad.data_ptr() % 16 != 0
    assert_exact(host(B.ternary_gemm_s8(Ad, Wd)), oracle.fwd(A, Wp), "fwd misaligned")
    dC = synth.uniform_int8(offset, 2, M, N)
    assert_exact(host(B.ternary_gemm_s8_dx(offset_view(dC, offset), Wd, K)),
                 oracle.dx(dC, Wp, K), "dx misaligned")
    assert_exact(host(B.ternary_gemm_s8_dw(Ad, offset_view(dC, offset))),
                 oracle.dw(A, dC), "dw misaligned")


@pytest.mark.parametrize("op,M,N,K", [("fwd", 300, 272, 96), ("fwd", 4100, 1900, 80),
                                      ("fwd", 27, 4099, 2112), ("fwd", 8197, 3000, 1536),
                                      ("dx", 299, 100, 268),
                                      ("dx", 27, 640, 1296),
                                      ("dw", 97, 271, 299)])
def test_writes_exactly_the_output(op, M, N, K):
    # the output sits between two canary bands inside one buffer, pre-filled
    # with a sentinel no result here can take; afterwards every output element
    # is written and no canary changed
    say(f"canary {op} {M}x{N}x{K}")
    R, Cc = {"fwd": (M, N), "dx": (M, K), "dw": (K, N)}[op]
    band = 4096 + 3
    sentinel, canary = 0x7FFFFFFF, -0x2A2A2A2B
    buf = torch.full((band + R * Cc + band,), canary, dtype=torch.int32, device=DEV)
    out = buf[band:band + R * Cc].view(R, Cc)
    out.fill_(sentinel)
    if op == "fwd":
        A, Wp = synth.fwd_inputs(9, M, N, K, 4)
        B.ternary_gemm_s8(dev(A), dev(Wp), C=out)
        want = oracle.fwd(A, Wp)
    elif op == "dx":
        dC, Wp = synth.dx_inputs(9, M, N, K, 4)
        B.ternary_gemm_s8_dx(dev(dC), dev(Wp), K, dX=out)
        want = oracle.dx(dC, Wp, K)
    else:
        A, dC = synth.dw_inputs(9, M, N, K)
        B.ternary_gemm_s8_dw(dev(A), dev(dC), dW=out)
        want = oracle.dw(A, dC)
    b = host(buf)
    assert (b[:band] == canary).all() and (b[band + R * Cc:] == canary).all()
    assert not (b[band:band + R * Cc] == sentinel).any()
    assert_exact(b[band:band + R * Cc].reshape(R, Cc), want, "canary case")


def test_deterministic_and_stream_independent():
    c = synth.CONFIGS["backward"]
    M, N, K = c["M"], c["N"], c["K"]
    say("determinism")
    A, Wp = synth.fwd_inputs(5, M, N, K, 3)
    Ad, Wd = dev(A), dev(Wp)
    first = B.ternary_gemm_s8(Ad, Wd).clone()
    s = torch.cuda.Stream()
    for _ in range(3):
        again = B.ternary_gemm_s8(Ad, Wd)
        assert torch.equal(first, again)
    with torch.cuda.stream(s):
        other = B.ternary_gemm_s8(Ad, Wd, stream=s)
    s.synchronize()
    assert torch.equal(first, other)


def test_shape_errors_raise():
    A = torch.zeros((4, 16), dtype=torch.int8, device=DEV)
    with pytest.raises(ValueError):
        B.ternary_gemm_s8(A, torch.zeros((4, 5), dtype=torch.uint8, device=DEV))
    A6 = torch.zeros((4, 6), dtype=torch.int8, device=DEV)
    W1 = torch.zeros((4, 2), dtype=torch.uint8, device=DEV)
    C = torch.zeros((4, 4), dtype=torch.int32, device=DEV)
    assert B.call_raw("ternary_gemm_s8", A6.data_ptr(), W1.data_ptr(), C.data_ptr(), 4, 4, 6) == B.ERR_PACK
    assert B.call_raw("ternary_gemm_s8", A6.data_ptr(), W1.data_ptr(), A6.data_ptr(), 4, 4, 4) == B.ERR_ALIAS


# ---------------------------------------------------------------------------
# scaled outputs: the integer product times per-row and per-column scales,
# stored as float32 or bfloat16; compared bit for bit with the oracle's
# integer result scaled the same way (IEEE single precision, nearest-even
# rounding, then nearest-even bfloat16)
# ---------------------------------------------------------------------------

SCALED_CASES = [
    ("fwd", 16384, 3456, 1280),   # stream kernel, the timed shape (every element)
    ("fwd", 16300, 3450, 640),    # stream kernel, ragged tiles, N % 4 != 0 (element stores)
    ("fwd", 4096, 4608, 64),      # stream kernel, one step per tile
    ("fwd", 15000, 3460, 192),    # stream kernel, N % 8 == 4: bf16 in 8-byte stores
    ("fwd", 300, 272, 96),        # tiled kernel
    ("fwd", 299, 271, 100),       # tiled kernel, guarded loads
    ("fwd", 27, 16384, 16384),    # skinny kernel, the skinny workload
    ("fwd", 32, 4099, 2112),      # skinny kernel, ragged columns (element stores)
    ("fwd", 5, 8200, 4160),       # skinny kernel, one 16-row block
    ("dx", 16300, 3456, 1296),    # stream dX, ragged rows and columns
    ("dx", 300, 96, 272),         # tiled dX
    ("dx", 27, 3456, 1280),       # skinny dX, the pages' 27 rows
    ("dx", 5, 8192, 8192),        # skinny dX, 64-column blocks, one 16-row block
    ("dx", 1782, 3456, 1280),     # dX, contraction split between two halves of a workgroup
    ("dw", 1090, 912, 4112),      # split dW kernel
    ("dw", 97, 271, 299),         # tiled dW, ragged
    ("dw", 16384, 3456, 1280),    # the timed shape
]
_int_results = {}


def _scaled_case(op, M, N, K):
    key = (op, M, N, K)
    seed = M + 3 * N + 5 * K
    if op == "fwd":
        A, Wp = synth.fwd_inputs(seed, M, N, K, 3)
        ins = (A, Wp)
        R, C = M, N
    elif op == "dx":
        dC, Wp = synth.dx_inputs(seed, M, N, K, 3)
        ins = (dC, Wp)
        R, C = M, K
    else:
        ins = synth.dw_inputs(seed, M, N, K)
        R, C = K, N
    rs = synth.positive_scales(seed, synth.STREAM_ROW_SCALE, R)
    cs = (synth.positive_scales(seed, synth.STREAM_COL_SCALE, C) if op == "dw"
          else np.float32(synth.W_SCALE))
    if key not in _int_results:
        _int_results.clear()
        _int_results[key] = (oracle.fwd(*ins) if op == "fwd" else
                             oracle.dx(ins[0], ins[1], K) if op == "dx" else oracle.dw(*ins))
    return ins, rs, cs, _int_results[key]


def _gpu_scaled(op, ins, K, rs, cs, dtype, out=None):
    if op == "fwd":
        return B.ternary_gemm_s8_scaled(dev(ins[0]), dev(ins[1]), dev(rs), float(cs), dtype, Y=out)
    if op == "dx":
        return B.ternary_gemm_s8_dx_scaled(dev(ins[0]), dev(ins[1]), K, dev(rs), float(cs), dtype, dX=out)
    return B.ternary_gemm_s8_dw_scaled(dev(ins[0]), dev(ins[1]), dev(rs), dev(cs), dtype, dW=out)


def _bits(t):
    torch = _torch_mod()
    return host(t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32))


def _torch_mod():
    import torch
    return torch


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("op,M,N,K", SCALED_CASES)
def test_scaled_outputs(op, M, N, K, kind):
    torch = _torch_mod()
    say(f"scaled {kind} {op} {M}x{N}x{K} plan={tile_of(op, M, N, K)}")
    ins, rs, cs, acc = _scaled_case(op, M, N, K)
    want = oracle.scale_output(acc, rs, cs, kind)
    dtype = torch.float32 if kind == "f32" else torch.bfloat16
    got = _bits(_gpu_scaled(op, ins, K, rs, cs, dtype))
    want_bits = want.view(np.int32) if kind == "f32" else want.view(np.int16)
    assert_exact(got, want_bits, f"scaled {kind} {op} {M}x{N}x{K}")


@pytest.mark.parametrize("op,M,N,K", [("fwd", 4096, 4608, 64), ("dx", 300, 96, 272), ("dw", 97, 271, 299)])
def test_scaled_output_misaligned(op, M, N, K):
    # a bf16 output starting 2 bytes into its buffer takes the element stores;
    # the bytes around it stay untouched
    torch = _torch_mod()
    say(f"scaled bf16 misaligned {op} {M}x{N}x{K}")
    ins, rs, cs, acc = _scaled_case(op, M, N, K)
    R, C = acc.shape
    buf = torch.full((R * C + 2,), -7, dtype=torch.int16, device=DEV)
    out = buf[1:1 + R * C].view(torch.bfloat16).view(R, C)
    _gpu_scaled(op, ins, K, rs, cs, torch.bfloat16, out=out)
    b = host(buf)
    assert b[0] == -7 and b[-1] == -7
    assert_exact(b[1:1 + R * C].reshape(R, C), oracle.scale_output(acc, rs, cs, "bf16").view(np.int16),
                 f"scaled misaligned {op}")


# ---------------------------------------------------------------------------
# the scaled outputs' reading, pinned on the GPU: acc values and scales chosen
# so that RN(RN(acc * rs) * cs) differs from RN(acc * RN(rs * cs)) are placed
# in chosen output elements of every kernel path; those elements must equal
# the exact binary32 model (tests/exact_f32.py) and every element the oracle
# ---------------------------------------------------------------------------

READING_SHAPES = [("fwd", 16, 100, 64), ("fwd", 300, 272, 96), ("fwd", 4096, 4608, 64),
                  ("dx", 27, 3456, 1280), ("dx", 300, 96, 272), ("dx", 16300, 3456, 1296),
                  ("dw", 97, 271, 299), ("dw", 1090, 912, 4112)]


def _reading_case(op, M, N, K):
    """Inputs whose exact product holds case i's acc at output (i, 0) (forward,
    dX) or (i, i) (dW), with random values everywhere else."""
    from test_oracle import SCALE_ORDER_CASES
    accs = [c[0] for c in SCALE_ORDER_CASES]
    seed = 7 + M + N + K
    if op == "fwd":
        A, Wp = synth.fwd_inputs(seed, M, N, K, 3)
        Wp[0, :] = 0
        Wp[0, 0] = 0x01                 # column 0: weight +1 at k = 0 only
        for i, v in enumerate(accs):
            A[i, 0] = v
        return (A, Wp), [(i, 0) for i in range(len(accs))]
    if op == "dx":
        dC, Wp = synth.dx_inputs(seed, M, N, K, 3)
        Wp[:, 0] &= 0xFC                # weight 0 at k = 0 in every row n ...
        Wp[0, 0] |= 0x01                # ... but +1 in row n = 0
        for i, v in enumerate(accs):
            dC[i, 0] = v
        return (dC, Wp), [(i, 0) for i in range(len(accs))]
    A, dC = synth.dw_inputs(seed, M, N, K)
    for i, v in enumerate(accs):
        A[:, i] = 0
        A[0, i] = 1                     # column i of A picks row 0 of dC
        dC[0, i] = v
    return (A, dC), [(i, i) for i in range(len(accs))]


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("op,M,N,K", READING_SHAPES)
def test_scaled_reading_exact_cases(op, M, N, K, kind):
    import exact_f32 as X
    from test_oracle import SCALE_ORDER_CASES
    torch = _torch_mod()
    say(f"scaled reading {kind} {op} {M}x{N}x{K} plan={tile_of(op, M, N, K)}")
    ins, spots = _reading_case(op, M, N, K)
    acc = oracle.fwd(*ins) if op == "fwd" else oracle.dx(ins[0], ins[1], K) if op == "dx" else oracle.dw(*ins)
    R, C = acc.shape
    dtype = torch.float32 if kind == "f32" else torch.bfloat16
    # the forward and dX take one column scale for the whole output: one call
    # per case; dW takes a scale per column: one call holds every case
    calls = [[i] for i in range(len(spots))] if op != "dw" else [list(range(len(spots)))]
    for cases in calls:
        rs = synth.positive_scales(R, synth.STREAM_ROW_SCALE, R)
        cs = synth.positive_scales(C, synth.STREAM_COL_SCALE, C) if op == "dw" else None
        for i in cases:
            acc_i, rb, cb = SCALE_ORDER_CASES[i]
            r, c = spots[i]
            assert int(acc[r, c]) == acc_i
            rs[r] = X.f32_of_bits(rb)
            if op == "dw":
                cs[c] = X.f32_of_bits(cb)
            else:
                cs = X.f32_of_bits(cb)
        got = _bits(_gpu_scaled(op, ins, K, rs, cs, dtype))
        want = oracle.scale_output(acc, rs, cs, kind)
        assert_exact(got, want.view(np.int32) if kind == "f32" else want.view(np.int16),
                     f"scaled reading {kind} {op} {M}x{N}x{K}")
        for i in cases:
            acc_i, rb, cb = SCALE_ORDER_CASES[i]
            r, c = spots[i]
            y = X.rn32(X.rn32(acc_i * X.exact(X.f32_of_bits(rb))) * X.exact(X.f32_of_bits(cb)))
            wb = X.bits32(y) if kind == "f32" else X.bits_bf16(X.rn_bf16(y))
            gb = int(got[r, c]) & (0xFFFFFFFF if kind == "f32" else 0xFFFF)
            assert gb == wb, (op, i, hex(gb), hex(wb))
