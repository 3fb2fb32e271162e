"""GPU parity of the steps before the product: the packer and the per-row /
per-column int8 quantizers against the oracle, bit for bit (stored bytes,
int8 values and float32 scale bit patterns), on the vector and the
element paths."""
import sys

import numpy as np
import pytest

import oracle
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


def assert_same(got, want, what):
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.argwhere(got != want)
    if len(bad):
        first = [(tuple(int(v) for v in ix), got[tuple(ix)], want[tuple(ix)]) for ix in bad[:8]]
        pytest.fail(f"{what}: {len(bad)} mismatches of {got.size}; first (index, gpu, oracle): {first}")


# ---------------------------------------------------------------------------
# packer
# ---------------------------------------------------------------------------

# (N, K): whole 64-byte chunks only, chunks plus a byte tail, bytes only, the
# benchmark's weights, and a large matrix
PACK_SHAPES = [(1, 4), (3, 12), (37, 96), (5, 260), (3456, 1280), (4096, 16384)]


@pytest.mark.parametrize("N,K", PACK_SHAPES)
def test_pack_ternary_weights(N, K):
    say(f"pack {N}x{K}")
    Wt = synth.ternary_int8(N + K, N, K)
    got = host(B.ternary_pack_weights(dev(Wt)))
    assert_same(got, oracle.pack_weights(Wt), f"pack {N}x{K}")


def test_pack_any_int8_by_sign():
    say("pack int8 by sign")
    W = synth.uniform_int8(3, synth.STREAM_A, 129, 320)
    assert_same(host(B.ternary_pack_weights(dev(W))), oracle.pack_weights(W), "pack by sign")


@pytest.mark.parametrize("offset", [1, 4])
def test_pack_misaligned(offset):
    # input and output starting inside their buffers take the byte kernel
    say(f"pack misaligned {offset}")
    N, K = 33, 200
    Wt = synth.ternary_int8(11, N, K)
    buf = torch.zeros(N * K + offset, dtype=torch.int8, device=DEV)
    buf[offset:] = dev(Wt).view(-1)
    out = torch.full((N * (K // 4) + offset + 1,), 0xA5, dtype=torch.uint8, device=DEV)
    B.ternary_pack_weights(buf[offset:].view(N, K), Wpacked=out[offset:offset + N * (K // 4)].view(N, K // 4))
    o = host(out)
    assert (o[:offset] == 0xA5).all() and o[-1] == 0xA5
    assert_same(o[offset:offset + N * (K // 4)].reshape(N, K // 4), oracle.pack_weights(Wt), "pack misaligned")


def test_pack_then_forward_matches_oracle():
    # the packed trainer weights feed the forward product unchanged
    say("pack -> forward")
    M, N, K = 300, 272, 96
    Wt = synth.ternary_int8(5, N, K)
    A = synth.uniform_int8(5, synth.STREAM_A, M, K)
    Wp = B.ternary_pack_weights(dev(Wt))
    C = host(B.ternary_gemm_s8(dev(A), Wp))
    want = A.astype(np.int64) @ Wt.astype(np.int64).T
    assert_same(C.astype(np.int64), want, "pack -> forward")


# ---------------------------------------------------------------------------
# quantizers
# ---------------------------------------------------------------------------

# (R, C): element path (C % 8 != 0), vector path, a row longer than one pass
# of the workgroup, the benchmark's activations
QUANT_SHAPES = [(1, 1), (3, 7), (300, 272), (65, 4104), (1782, 3456), (16384, 1280)]


def _input(R, C, kind):
    X = synth.float_inputs(R * 3 + C, synth.STREAM_X, R, C, kind)
    if R >= 3:
        X[1] = 0                                             # an all-zero row
    return X


def _to_torch(X, kind):
    t = dev(X)
    return t if kind == "f32" else t.view(torch.bfloat16)


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("R,C", QUANT_SHAPES)
def test_quantize_rows(R, C, kind):
    say(f"quantize rows {kind} {R}x{C}")
    X = _input(R, C, kind)
    Q, S = B.ternary_quantize_rows(_to_torch(X, kind))
    q, s = oracle.quantize(X, kind, "rows")
    assert_same(host(S).view(np.uint32), s.view(np.uint32), "row scales")
    assert_same(host(Q), q, f"rows {kind} {R}x{C}")


@pytest.mark.parametrize("kind", ["f32", "bf16"])
@pytest.mark.parametrize("R,C", QUANT_SHAPES)
def test_quantize_cols(R, C, kind):
    say(f"quantize cols {kind} {R}x{C}")
    X = _input(R, C, kind)
    if C >= 3:
        X[:, 2] = 0                                          # an all-zero column
    Q, S = B.ternary_quantize_cols(_to_torch(X, kind))
    q, s = oracle.quantize(X, kind, "cols")
    assert_same(host(S).view(np.uint32), s.view(np.uint32), "column scales")
    assert_same(host(Q), q, f"cols {kind} {R}x{C}")


def test_quantize_ties_and_extremes():
    # s = 1 exactly (127 in the row), halves round to even, -127 .. 127
    say("quantize ties")
    x = np.array([[127, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5, -127, 0, -0.0, 1, 64.5, -64.5, 100, 7]],
                 dtype=np.float32)
    Q, S = B.ternary_quantize_rows(dev(x))
    assert host(S).tolist() == [1.0]
    assert host(Q).tolist() == [[127, 2, 4, -2, -4, 0, 0, 126, -127, 0, 0, 1, 64, -64, 100, 7]]
    Qc, Sc = B.ternary_quantize_cols(dev(np.ascontiguousarray(x.T)))
    assert host(Sc).tolist() == [1.0] and host(Qc).T.tolist() == host(Q).tolist()


def test_quantize_then_scaled_forward():
    # quantized activations and their row scales feed the scaled forward: the
    # result is the oracle's scaled output of the oracle's quantized product
    say("quantize -> scaled forward")
    M, N, K = 300, 272, 96
    X = synth.float_inputs(9, synth.STREAM_X, M, K, "bf16")
    _, Wp = synth.fwd_inputs(9, M, N, K, 3)
    Q, S = B.ternary_quantize_rows(_to_torch(X, "bf16"))
    Y = B.ternary_gemm_s8_scaled(Q, dev(Wp), S, synth.W_SCALE, torch.float32)
    q, s = oracle.quantize(X, "bf16", "rows")
    want = oracle.scale_output(oracle.fwd(q, Wp), s, np.float32(synth.W_SCALE), "f32")
    assert_same(host(Y).view(np.uint32), want.view(np.uint32), "quantize -> scaled forward")


def test_quantize_misaligned_output():
    # an int8 output starting 1 byte into its buffer takes the element path;
    # the bytes around it stay untouched
    say("quantize misaligned")
    R, C = 40, 64
    X = _input(R, C, "f32")
    buf = torch.full((R * C + 2,), 77, dtype=torch.int8, device=DEV)
    Q, S = B.ternary_quantize_rows(dev(X), Q=buf[1:1 + R * C].view(R, C))
    b = host(buf)
    assert b[0] == 77 and b[-1] == 77
    assert_same(b[1:1 + R * C].reshape(R, C), oracle.quantize(X, "f32", "rows")[0], "misaligned")


@pytest.mark.parametrize("R,C", [(300, 272), (130, 37)])
def test_quantize_cols_misaligned_output(R, C):
    # an int8 output that is not 4-byte aligned cannot hold the per-run
    # partial maxima, so the column scales come from the atomic-max path
    say(f"quantize cols misaligned {R}x{C}")
    X = _input(R, C, "bf16")
    buf = torch.full((R * C + 2,), 77, dtype=torch.int8, device=DEV)
    Q, S = B.ternary_quantize_cols(_to_torch(X, "bf16"), Q=buf[1:1 + R * C].view(R, C))
    b = host(buf)
    q, s = oracle.quantize(X, "bf16", "cols")
    assert b[0] == 77 and b[-1] == 77
    assert_same(host(S).view(np.uint32), s.view(np.uint32), "column scales (atomic path)")
    assert_same(b[1:1 + R * C].reshape(R, C), q, "cols misaligned")


def test_grid_stride_paths():
    # more 64-byte chunks than the packer's grid has threads (8192 x 256), and
    # more rows than the row quantizer's grid has waves (524288 x 4): both
    # kernels loop over the remainder
    N, K = 8200, 16400
    say(f"pack grid-stride {N}x{K}")
    Wt = synth.ternary_int8(21, N, K)
    assert N * K // 64 > 8192 * 256
    assert_same(host(B.ternary_pack_weights(dev(Wt))), oracle.pack_weights(Wt), "pack grid-stride")
    del Wt
    R, C = 2_100_000, 8
    say(f"quantize rows grid-stride {R}x{C}")
    X = synth.float_inputs(22, synth.STREAM_X, R, C, "bf16")
    assert R > 524288 * 4
    Q, S = B.ternary_quantize_rows(_to_torch(X, "bf16"))
    q, s = oracle.quantize(X, "bf16", "rows")
    assert_same(host(S).view(np.uint32), s.view(np.uint32), "row scales grid-stride")
    assert_same(host(Q), q, "rows grid-stride")


def test_quantize_cols_grid_stride():
    # more 16-row groups than the column kernel's grid has in y (65535): its
    # workgroups loop over the remainder
    R, C = 1_100_000, 8
    say(f"quantize cols grid-stride {R}x{C}")
    assert -(-R // 16) > 65535
    X = synth.float_inputs(23, synth.STREAM_X, R, C, "bf16")
    Q, S = B.ternary_quantize_cols(_to_torch(X, "bf16"))
    q, s = oracle.quantize(X, "bf16", "cols")
    assert_same(host(S).view(np.uint32), s.view(np.uint32), "column scales grid-stride")
    assert_same(host(Q), q, "cols grid-stride")


@pytest.mark.parametrize("kind_path", ["elements", "vector"])
def test_quantize_exact_reading_cases(kind_path):
    # values chosen so that the division readings (s = RN(max / 127), q =
    # rint(RN(x / s))) differ from the reciprocal ones; scales and values must
    # equal the exact binary32 model (tests/exact_f32.py) and the oracle, on
    # rows and on columns
    from fractions import Fraction

    import exact_f32 as X
    from test_oracle import SCALE_DIVISION_CASES, VALUE_DIVISION_CASES
    say(f"quantize exact reading cases ({kind_path})")
    C = 3 if kind_path == "elements" else 64
    rows = []
    for mb in SCALE_DIVISION_CASES:
        m = X.f32_of_bits(mb)
        rows.append([m, -m / np.float32(3), np.float32(0.25)])
    for mb, xb in VALUE_DIVISION_CASES:
        rows.append([X.f32_of_bits(mb), X.f32_of_bits(xb), -X.f32_of_bits(xb)])
    x = np.zeros((len(rows), C), dtype=np.float32)
    x[:, :3] = np.array(rows, dtype=np.float32)
    for axis, xin in (("rows", x), ("cols", np.ascontiguousarray(x.T))):
        fn = B.ternary_quantize_rows if axis == "rows" else B.ternary_quantize_cols
        Q, S = fn(dev(xin))
        q, s = oracle.quantize(xin, "f32", axis)
        got_q, got_s = host(Q), host(S).view(np.uint32)
        assert_same(got_s, s.view(np.uint32), f"{axis} scales")
        assert_same(got_q, q, f"{axis} values")
        gq = got_q if axis == "rows" else got_q.T
        for r, vals in enumerate(rows):
            sr = X.rn32(max(abs(X.exact(v)) for v in vals) / 127)
            assert int(got_s[r]) == X.bits32(sr), (axis, r)
            want = [max(-127, min(127, X.round_half_even(X.rn32(X.exact(v) / sr)))) for v in vals]
            assert gq[r, :3].tolist() == want, (axis, r)
