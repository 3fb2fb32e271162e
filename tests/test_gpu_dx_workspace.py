"""GPU parity of dX with a workspace (the contraction split across workgroups
and the partials summed by a second kernel) against the oracle, bit for bit,
and against the one-pass call: int32 and both scaled kinds, reused and
undersized workspaces, misaligned workspaces and outputs."""
import sys

import numpy as np
import pytest

import oracle
from ternary_weight_int8_amd import binding as B
from ternary_weight_int8_amd import synth
from shapes import SPLIT_DX_SHAPES

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


def _inputs(M, N, K, alphabet=4):
    return synth.dx_inputs(M * 19 + N + 3 * K, M, N, K, alphabet)


@pytest.mark.parametrize("M,N,K", SPLIT_DX_SHAPES)
def test_split_dx_shapes(M, N, K):
    nbytes = B.ternary_gemm_dx_workspace(M, N, K)
    say(f"dx workspace {M}x{N}x{K} workspace={nbytes}")
    assert nbytes > 0
    dC, Wp = _inputs(M, N, K)
    dCd, Wd = dev(dC), dev(Wp)
    ws = torch.full((nbytes,), 0x5A, dtype=torch.uint8, device=DEV)   # garbage on entry
    got = host(B.ternary_gemm_s8_dx_ws(dCd, Wd, K, workspace=ws))
    assert_exact(got, oracle.dx(dC, Wp, K), f"dx workspace {M}x{N}x{K}")
    assert_exact(host(B.ternary_gemm_s8_dx(dCd, Wd, K)), got, f"one-pass vs split {M}x{N}x{K}")


def test_split_dx_extreme():
    # every dC entry -128 and every weight +1 (columns < 128) or -1: each
    # partial and the sum reach -128 N and 128 N exactly
    M, N, K = 2, 16384, 16384
    say(f"dx workspace extreme {M}x{N}x{K}")
    dC = np.full((M, N), -128, dtype=np.int8)
    codes = np.where(np.arange(K) < 128, 1, 2).astype(np.uint8)          # code 1: +1, 2: -1
    row = (codes[0::4] | (codes[1::4] << 2) | (codes[2::4] << 4) | (codes[3::4] << 6)).astype(np.uint8)
    Wp = np.tile(row, (N, 1))
    got = host(B.ternary_gemm_s8_dx_ws(dev(dC), dev(Wp), K))
    assert (got[:, :128] == -128 * N).all() and (got[:, 128:] == 128 * N).all()
    assert_exact(got, oracle.dx(dC, Wp, K), "dx workspace extreme vs oracle")


def test_workspace_reused_then_smaller_call():
    # one workspace for two calls in a row, the second smaller: the second
    # call's partials overwrite what it reads, so stale contents never leak
    big, small = (27, 16384, 16384), (3, 6400, 12800)
    nbytes = B.ternary_gemm_dx_workspace(*big)
    assert B.ternary_gemm_dx_workspace(*small) < nbytes
    ws = torch.empty(nbytes, dtype=torch.uint8, device=DEV)
    for M, N, K in (big, small, big):
        say(f"dx workspace reuse {M}x{N}x{K}")
        dC, Wp = _inputs(M, N, K, 3)
        got = host(B.ternary_gemm_s8_dx_ws(dev(dC), dev(Wp), K, workspace=ws))
        assert_exact(got, oracle.dx(dC, Wp, K), f"dx workspace reuse {M}x{N}x{K}")


@pytest.mark.parametrize("how", ["too small", "misaligned"])
def test_unusable_workspace_runs_one_pass(how):
    # a workspace one byte short, or not 16-byte aligned, is not used: the
    # one-pass kernel runs and leaves the workspace as it was
    M, N, K = 16, 4096, 8192
    say(f"dx workspace {how}")
    nbytes = B.ternary_gemm_dx_workspace(M, N, K)
    buf = torch.full((nbytes + 16,), 0x33, dtype=torch.uint8, device=DEV)
    ws = buf[: nbytes - 1] if how == "too small" else buf[4: 4 + nbytes]
    dC, Wp = _inputs(M, N, K)
    got = host(B.ternary_gemm_s8_dx_ws(dev(dC), dev(Wp), K, workspace=ws))
    assert_exact(got, oracle.dx(dC, Wp, K), f"dx workspace {how}")
    assert (host(buf) == 0x33).all()


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("M,N,K", [(27, 16384, 16384), (16, 4096, 8192)])
def test_split_dx_scaled(M, N, K, kind):
    say(f"dx workspace scaled {kind} {M}x{N}x{K}")
    dC, Wp = _inputs(M, N, K, 3)
    rs = synth.positive_scales(M + K, synth.STREAM_ROW_SCALE, M)
    dtype = torch.float32 if kind == "f32" else torch.bfloat16
    itype = torch.int32 if kind == "f32" else torch.int16
    dCd, Wd, rsd = dev(dC), dev(Wp), dev(rs)
    got = host(B.ternary_gemm_s8_dx_scaled_ws(dCd, Wd, K, rsd, synth.W_SCALE, dtype).view(itype))
    want = oracle.scale_output(oracle.dx(dC, Wp, K), rs, np.float32(synth.W_SCALE), kind)
    assert_exact(got, want.view(np.int32 if kind == "f32" else np.int16), f"dx workspace scaled {kind}")
    one = host(B.ternary_gemm_s8_dx_scaled(dCd, Wd, K, rsd, synth.W_SCALE, dtype).view(itype))
    assert_exact(one, got, f"one-pass vs split scaled {kind}")


@pytest.mark.parametrize("kind", ["i32", "bf16"])
def test_split_dx_misaligned_output(kind):
    # an output starting one element into its buffer takes the summing
    # kernel's element stores; the elements around it stay untouched
    M, N, K = 5, 4096, 8192
    say(f"dx workspace misaligned output {kind}")
    dC, Wp = _inputs(M, N, K, 3)
    acc = oracle.dx(dC, Wp, K)
    if kind == "i32":
        buf = torch.full((M * K + 2,), -7, dtype=torch.int32, device=DEV)
        B.ternary_gemm_s8_dx_ws(dev(dC), dev(Wp), K, dX=buf[1:1 + M * K].view(M, K))
        want = acc
    else:
        rs = synth.positive_scales(7, synth.STREAM_ROW_SCALE, M)
        buf = torch.full((M * K + 2,), -7, dtype=torch.int16, device=DEV)
        out = buf[1:1 + M * K].view(torch.bfloat16).view(M, K)
        B.ternary_gemm_s8_dx_scaled_ws(dev(dC), dev(Wp), K, dev(rs), synth.W_SCALE, torch.bfloat16, dX=out)
        want = oracle.scale_output(acc, rs, np.float32(synth.W_SCALE), "bf16").view(np.int16)
    b = host(buf)
    assert b[0] == -7 and b[-1] == -7
    assert_exact(b[1:1 + M * K].reshape(M, K), want, f"dx workspace misaligned {kind}")


def test_concurrent_calls_with_their_own_workspaces():
    # two streams, each with its own workspace, run the split dX at the same
    # time on different shapes; both results match the oracle
    shapes = [(27, 16384, 16384), (16, 4096, 8192)]
    say("dx workspace on two streams")
    ins = [_inputs(M, N, K, 3) for (M, N, K) in shapes]
    devs = [(dev(dC), dev(Wp)) for (dC, Wp) in ins]
    wss = [torch.empty(B.ternary_gemm_dx_workspace(*s), dtype=torch.uint8, device=DEV) for s in shapes]
    outs = [torch.empty((M, K), dtype=torch.int32, device=DEV) for (M, N, K) in shapes]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    want = [oracle.dx(dC, Wp, K) for (dC, Wp), (M, N, K) in zip(ins, shapes)]
    torch.cuda.synchronize()
    for rep in range(3):
        for i, (M, N, K) in enumerate(shapes):
            B.ternary_gemm_s8_dx_ws(devs[i][0], devs[i][1], K, workspace=wss[i], dX=outs[i], stream=streams[i])
        torch.cuda.synchronize()
        for i, (M, N, K) in enumerate(shapes):
            assert_exact(host(outs[i]), want[i], f"stream {i} rep {rep} {M}x{N}x{K}")
