"""The dX entry point that allocates nothing (ternary_gemm_s8_dx_noalloc),
called through the C ABI with caller-allocated tensors, against the
workspace entry point ternary_gemm_s8_dx_ws on the same inputs, bit for bit:
two calls in a row (the second smaller, so the static scratch holds the
first call's partial sums when it starts), a shape without a split, and the
rejection of a split that needs more scratch than the static buffer."""
import ctypes
import sys

import numpy as np
import pytest

from ternary_weight_int8_amd import binding as B
from ternary_weight_int8_amd import synth

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(seed, M, N, K):
    dC, Wp = synth.dx_inputs(seed, M, N, K, 3)
    return torch.from_numpy(dC).to(DEV), torch.from_numpy(Wp).to(DEV)


def _with_workspace(dC, Wp, M, N, K):
    nbytes = B.ternary_gemm_dx_workspace(M, N, K, 256)
    ws = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=DEV)
    out = torch.empty((M, K), dtype=torch.int32, device=DEV)
    st = B.lib().ternary_gemm_s8_dx_ws(dC.data_ptr(), Wp.data_ptr(), out.data_ptr(), M, N, K, ws.data_ptr(),
                                       ws.numel(), None)
    assert st == B.OK, B.status_str(st)
    return out, nbytes


def _noalloc(dC, Wp, out, M, N, K):
    return B.lib().ternary_gemm_s8_dx_noalloc(dC.data_ptr(), Wp.data_ptr(), out.data_ptr(), M, N, K, None)


@pytest.mark.parametrize("M,N,K,split", [
    (27, 16384, 16384, True),    # the pages' 27 rows at 16384^2: 4 splits, 7 MB of partial sums
    (5, 4096, 8192, True),       # smaller: 8 splits over the previous call's partial sums
    (40, 4096, 2048, False),     # more than 32 rows: no split, the one-pass kernels
])
def test_noalloc_matches_workspace_call(M, N, K, split):
    say(f"noalloc dX {M}x{N}x{K}")
    dC, Wp = _inputs(M + N + K, M, N, K)
    ref, nbytes = _with_workspace(dC, Wp, M, N, K)
    assert (nbytes > 0) == split and nbytes <= B.STATIC_SCRATCH_BYTES
    for rep in range(2):
        out = torch.full((M, K), -7, dtype=torch.int32, device=DEV)
        st = _noalloc(dC, Wp, out, M, N, K)
        assert st == B.OK, B.status_str(st)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), (M, N, K, rep)


def test_noalloc_two_calls_in_a_row():
    # the second call is smaller and starts on the first call's partial sums
    a = (27, 16384, 16384)
    b = (3, 6400, 12800)
    ins = {s: _inputs(7 + sum(s), *s) for s in (a, b)}
    refs = {s: _with_workspace(*ins[s], *s)[0] for s in (a, b)}
    outs = {s: torch.empty((s[0], s[2]), dtype=torch.int32, device=DEV) for s in (a, b)}
    say("noalloc dX: two calls in a row")
    for s in (a, b):
        assert _noalloc(*ins[s], outs[s], *s) == B.OK
    torch.cuda.synchronize()
    for s in (a, b):
        assert torch.equal(outs[s], refs[s]), s


def test_noalloc_rejects_a_split_past_the_static_buffer():
    # 32 rows x K = 21760: 85 column blocks, 4 splits, 4 * 32 * 21760 * 4
    # bytes (11.1 MB) of partial sums, more than the 8 MiB buffer
    M, N, K = 32, 2048, 21760
    nbytes = B.ternary_gemm_dx_workspace(M, N, K, 256)
    assert nbytes > B.STATIC_SCRATCH_BYTES, nbytes
    dC, Wp = _inputs(5, M, N, K)
    out = torch.full((M, K), -7, dtype=torch.int32, device=DEV)
    say(f"noalloc dX past the buffer {M}x{N}x{K}")
    assert _noalloc(dC, Wp, out, M, N, K) == B.ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((out == -7).all())     # nothing launched
    with pytest.raises(B.TernaryGemmError):
        B.ternary_gemm_s8_dx_noalloc(dC, Wp, K)


def test_noalloc_inside_a_captured_graph():
    # the callers it is for: code under graph capture.  Captured once after an
    # eager call, replayed three times with eager work between the replays,
    # every replay equal to the eager result
    M, N, K = 27, 8192, 8192
    dC, Wp = _inputs(11, M, N, K)
    out = torch.empty((M, K), dtype=torch.int32, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.ternary_gemm_s8_dx_noalloc(dC, Wp, K, dX=out, stream=side)
    side.synchronize()
    eager = out.clone()
    ref, nbytes = _with_workspace(dC, Wp, M, N, K)
    assert nbytes > 0 and torch.equal(eager, ref)
    say(f"noalloc dX in a graph {M}x{N}x{K}")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        B.ternary_gemm_s8_dx_noalloc(dC, Wp, K, dX=out, stream=side)
    other = _inputs(12, 5, 4096, 8192)
    for rep in range(3):
        out.zero_()
        # eager no-alloc work between the replays, on the same static scratch
        junk = torch.empty((5, 8192), dtype=torch.int32, device=DEV)
        assert _noalloc(*other, junk, 5, 4096, 8192) == B.OK
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {rep} differs from the eager result"
