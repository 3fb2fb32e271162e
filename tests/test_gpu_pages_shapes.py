"""GPU parity on the pages' own shape lists, every element against the oracle.

* The forward shapes reported bit-exact on the pages (t27 pull request
  #10425, results comment "RTX 4090 run", table "Bit-exact"), read from
  tests/golden/bitexact_shapes.txt.
* The HSLM backward shapes (t27 pull request #10855, commit message and
  "Measured: RTX 4090"): every HSLM shape at 27 and 1782 rows, layer widths
  243 and 729, which the pages pad to the kernels' multiple of 16 (256, 736).
  Here the stored (packed) dimension, the layer input K, takes the padded
  widths, since the packed layout needs K % 4 == 0 and 243 and 729 are not;
  the other dimensions run at both the true and the padded widths.
"""
import sys

import numpy as np
import pytest

import oracle
from golden_io import read_rows
from ternary_weight_int8_amd import binding as B
from ternary_weight_int8_amd import synth

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


def plan_of(op, M, N, K):
    return B.plan(op, M, N, K).kernel


BITEXACT = read_rows("bitexact_shapes.txt")


def test_bitexact_table_is_the_pages():
    # the fixture holds the table's nine shapes, brace rows expanded
    assert len(BITEXACT) == 9
    assert (300, 272, 96) in BITEXACT and (16384, 3456, 1280) in BITEXACT


@pytest.mark.parametrize("M,N,K", BITEXACT)
def test_pages_bitexact_shapes(M, N, K):
    # codes over {0,1,2,3} on the small shapes (code 3 is the second zero),
    # {0,1,2} on the "500m" shapes, as the workloads draw them
    alphabet = 4 if M * N <= 300 * 272 else 3
    seed = (M * 31 + N * 7 + K) % 1000
    say(f"pages bit-exact {M}x{N}x{K} seed={seed} plan={plan_of('fwd', M, N, K)}")
    A, Wp = synth.fwd_inputs(seed, M, N, K, alphabet)
    C = host(B.ternary_gemm_s8(dev(A), dev(Wp)))
    assert_exact(C, oracle.fwd(A, Wp), f"forward {M}x{N}x{K}")


HSLM_ROWS = (27, 1782)
HSLM_PACKED = (256, 736)               # layer input K: the padded widths
HSLM_OTHER = (243, 729, 256, 736)      # layer output N: true and padded widths
HSLM_FWD_DX = [(M, N, K) for M in HSLM_ROWS for K in HSLM_PACKED for N in HSLM_OTHER]
HSLM_DW = [(M, N, K) for M in HSLM_ROWS
           for (K, N) in [(243, 243), (243, 729), (729, 243), (729, 729),
                          (256, 256), (256, 736), (736, 256), (736, 736)]]


@pytest.mark.parametrize("M,N,K", HSLM_FWD_DX)
def test_hslm_forward(M, N, K):
    seed = M + N + K
    say(f"hslm forward {M}x{N}x{K} plan={plan_of('fwd', M, N, K)}")
    A, Wp = synth.fwd_inputs(seed, M, N, K, 3)
    assert_exact(host(B.ternary_gemm_s8(dev(A), dev(Wp))), oracle.fwd(A, Wp), f"hslm fwd {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", HSLM_FWD_DX)
def test_hslm_dx(M, N, K):
    seed = 2 * M + N + K
    say(f"hslm dX {M}x{N}x{K} plan={plan_of('dx', M, N, K)}")
    dC, Wp = synth.dx_inputs(seed, M, N, K, 3)
    assert_exact(host(B.ternary_gemm_s8_dx(dev(dC), dev(Wp), K)), oracle.dx(dC, Wp, K),
                 f"hslm dX {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", HSLM_DW)
def test_hslm_dw(M, N, K):
    seed = 3 * M + N + K
    say(f"hslm dW {M}x{N}x{K} plan={plan_of('dw', M, N, K)}")
    A, dC = synth.dw_inputs(seed, M, N, K)
    assert_exact(host(B.ternary_gemm_s8_dw(dev(A), dev(dC))), oracle.dw(A, dC), f"hslm dW {M}x{N}x{K}")
