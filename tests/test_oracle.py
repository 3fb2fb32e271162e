"""Pins for the CPU oracle (no GPU).

The oracle is checked here against what the pages and plain mathematics fix,
never against itself: the byte table printed on the pages, hand-computed
products, closed forms, exact extremes at the int32 bound, and numpy's int64
matmul (a library routine) over a decode written separately from the page's
byte table.  Each group below names the mistake it is there to catch.
"""
from fractions import Fraction

import numpy as np
import pytest

import exact_f32 as X
import oracle
from golden_io import read_kv
from ternary_weight_int8_amd import synth


def page_table_weights():
    """int8 weight of codes 0..3, read from the page's byte-permute table."""
    t = read_kv("decode_table.txt")["perm_table"]
    return np.array([(t >> (8 * c)) & 0xFF for c in range(4)], dtype=np.uint8).view(np.int8)


def lut_decode(codes):
    """Separate decode for the brute-force checks: page table indexed by code."""
    return page_table_weights()[codes.astype(np.intp)]


def codes_of_bytes_lsb_first(b):
    """2-bit fields of each byte, first field in the low bits."""
    b = np.asarray(b, dtype=np.uint8)
    return np.stack([(b >> (2 * i)) & 3 for i in range(4)], axis=-1)


# -- decode table (catches: wrong sign, code 3 treated as nonzero) ---------------

def test_page_table_is_the_formula_table():
    # two independent statements on the pages agree: 0,+1,-1,0
    assert page_table_weights().tolist() == [0, 1, -1, 0]


def test_oracle_weight_of_code_matches_page_table():
    assert [oracle.weight_of_code(c) for c in range(4)] == page_table_weights().tolist()


def test_decode_every_byte_matches_page_table():
    Wp = np.arange(256, dtype=np.uint8).reshape(256, 1)       # N=256 rows, K=4
    got = oracle.decode(Wp, 4)
    want = lut_decode(codes_of_bytes_lsb_first(np.arange(256)))
    np.testing.assert_array_equal(got, want)


# -- packing (catches: bit order, row stride) -----------------------------------

@pytest.mark.parametrize("byte,weights", [
    (0x00, [0, 0, 0, 0]),
    (0x01, [1, 0, 0, 0]),
    (0x02, [-1, 0, 0, 0]),
    (0x04, [0, 1, 0, 0]),
    (0x40, [0, 0, 0, 1]),
    (0x80, [0, 0, 0, -1]),
    (0x06, [-1, 1, 0, 0]),
    (0x55, [1, 1, 1, 1]),
    (0xAA, [-1, -1, -1, -1]),
    (0xFF, [0, 0, 0, 0]),
    (0xC9, [1, -1, 0, 0]),
])
def test_hand_bytes(byte, weights):
    got = oracle.decode(np.array([[byte]], dtype=np.uint8), 4)
    assert got.tolist() == [weights]


def test_pack_unpack_roundtrip_all_bytes():
    Wp = np.arange(256, dtype=np.uint8).reshape(16, 16)       # N=16, K=64
    codes = oracle.unpack(Wp, 64)
    assert codes.max() <= 3
    np.testing.assert_array_equal(oracle.pack(codes), Wp)


def test_unpack_pack_roundtrip_random_codes():
    rng = np.random.default_rng(7)
    codes = rng.integers(0, 4, size=(37, 52), dtype=np.uint8)
    np.testing.assert_array_equal(oracle.unpack(oracle.pack(codes), 52), codes)


def test_row_stride_is_k_over_4():
    # code (k, n) lives in byte n*(K/4) + k/4
    N, K = 3, 12
    codes = np.zeros((N, K), dtype=np.uint8)
    codes[2, 9] = 1
    Wp = oracle.pack(codes).reshape(-1)
    assert np.flatnonzero(Wp).tolist() == [2 * (K // 4) + 9 // 4]
    assert Wp[2 * 3 + 2] == 1 << (2 * (9 % 4))


def test_generator_placement_agrees_with_oracle_pack():
    codes = synth.random_codes(3, 29, 40, 4)
    np.testing.assert_array_equal(synth.store_codes(codes), oracle.pack(codes))


# -- forward: hand cases (catches: dropped term, transposed operand) ------------

def test_fwd_hand_1x1x4():
    # A = [3, -5, 7, 100]; codes 1, 2, 0, 3 -> weights +1, -1, 0, 0 -> 3 + 5 = 8
    A = np.array([[3, -5, 7, 100]], dtype=np.int8)
    Wp = np.array([[0xC9]], dtype=np.uint8)
    assert oracle.fwd(A, Wp).tolist() == [[8]]


def test_fwd_hand_2x3x8():
    A = np.array([[1, 2, 3, 4, 5, 6, 7, 8],
                  [-1, -2, -3, -4, -5, -6, -7, -8]], dtype=np.int8)
    # n=0: all +1                       -> 36
    # n=1: -1,-1,-1,-1, 0,0,0,0        -> -(1+2+3+4) = -10
    # n=2: +1,-1,+1,-1, 0,0,0,0 (code 3) -> 1-2+3-4 = -2
    Wp = np.array([[0x55, 0x55],
                   [0xAA, 0x00],
                   [0x99, 0xFF]], dtype=np.uint8)
    assert oracle.fwd(A, Wp).tolist() == [[36, -10, -2], [-36, 10, 2]]


# -- forward: closed forms -------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(1, 1, 4), (3, 5, 64), (7, 2, 1000)])
def test_fwd_ones_times_plus_one_is_K(M, N, K):
    A = np.ones((M, K), dtype=np.int8)
    Wp = np.full((N, K // 4), 0x55, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.fwd(A, Wp), np.full((M, N), K))


@pytest.mark.parametrize("byte,scale", [(0x55, -128), (0xAA, 128), (0x00, 0), (0xFF, 0)])
def test_fwd_minus128_closed_forms(byte, scale):
    M, N, K = 2, 3, 256
    A = np.full((M, K), -128, dtype=np.int8)
    Wp = np.full((N, K // 4), byte, dtype=np.uint8)
    np.testing.assert_array_equal(oracle.fwd(A, Wp), np.full((M, N), scale * K))


def test_fwd_swap_codes_negates():
    A = synth.uniform_int8(11, 0, 9, 48)
    codes = synth.random_codes(11, 7, 48, 4)
    swapped = codes.copy()
    swapped[codes == 1] = 2
    swapped[codes == 2] = 1
    C = oracle.fwd(A, synth.store_codes(codes))
    Cs = oracle.fwd(A, synth.store_codes(swapped))
    np.testing.assert_array_equal(Cs, -C)


def test_fwd_row_sum_identity():
    # sum_n C[m][n] = sum_k A[m][k] * (sum_n w(k, n))
    A = synth.uniform_int8(5, 0, 6, 40)
    codes = synth.random_codes(5, 9, 40, 4)
    C = oracle.fwd(A, synth.store_codes(codes)).astype(np.int64)
    colsum = lut_decode(codes).astype(np.int64).sum(axis=0)          # over n -> [K]
    want = (A.astype(np.int64) * colsum[None, :]).sum(axis=1)
    np.testing.assert_array_equal(C.sum(axis=1), want)


# -- forward: brute force against numpy int64 matmul ------------------------------

def test_fwd_exhaustive_code_columns():
    # K=4, every one of the 256 possible code columns, A rows with the extremes
    A = np.array([[-128, -128, -128, -128], [127, 127, 127, 127], [-128, 127, -1, 0],
                  [1, 2, 3, 4], [0, 0, 0, 0], [-7, 19, -64, 99],
                  [127, -128, 127, -128], [5, -5, 5, -5]], dtype=np.int8)
    codes = codes_of_bytes_lsb_first(np.arange(256)).astype(np.uint8)   # [256][4]
    Wp = np.arange(256, dtype=np.uint8).reshape(256, 1)
    want = A.astype(np.int64) @ lut_decode(codes).astype(np.int64).T
    np.testing.assert_array_equal(oracle.fwd(A, Wp), want)


@pytest.mark.parametrize("M,N,K,alphabet,seed", [
    (1, 16, 16, 4, 1), (5, 3, 8, 4, 2), (17, 33, 96, 4, 3), (64, 7, 132, 3, 4), (2, 130, 260, 3, 5)])
def test_fwd_brute_force(M, N, K, alphabet, seed):
    A = synth.uniform_int8(seed, 0, M, K)
    codes = synth.random_codes(seed, N, K, alphabet)
    want = A.astype(np.int64) @ lut_decode(codes).astype(np.int64).T
    np.testing.assert_array_equal(oracle.fwd(A, synth.store_codes(codes), threads=3), want)


# -- forward: the int32 extremes (catches: int32 accumulation, missing overflow check)

def test_fwd_int32_extremes_at_bound():
    K = 16777212                            # largest multiple of 4 under 2^31/128
    assert K <= read_kv("bounds.txt")["ternary_max_contraction"] < K + 4
    A = np.full((1, K), -128, dtype=np.int8)
    Wp = np.empty((2, K // 4), dtype=np.uint8)
    Wp[0] = 0x55
    Wp[1] = 0xAA
    C, r = oracle.fwd(A, Wp, return_overflows=True)
    assert r == 0
    assert C.tolist() == [[-2147483136, 2147483136]]
    assert C[0, 0] == np.iinfo(np.int32).min + 512
    assert C[0, 1] == np.iinfo(np.int32).max - 511


def test_fwd_overflow_detected_past_bound():
    K = 1 << 24
    A = np.full((1, K), -128, dtype=np.int8)
    Wp = np.empty((2, K // 4), dtype=np.uint8)
    Wp[0] = 0x55                            # -2^31 exactly: representable
    Wp[1] = 0xAA                            # +2^31: not representable
    C, r = oracle.fwd(A, Wp, allow_overflow=True, return_overflows=True)
    assert r == 1
    assert C[0, 0] == np.iinfo(np.int32).min
    assert C[0, 1] == np.iinfo(np.int32).min   # wrapped low 32 bits of 2^31
    with pytest.raises(oracle.OverflowInOracle):
        oracle.fwd(A, Wp)


def test_fwd_structured_halves_closed_form():
    # the structured stress recipe, at a size the oracle does quickly
    M, N, K = 64, 48, 4096
    A, Wp = synth.extreme_inputs(2, M, N, K)
    C = oracle.fwd(A, Wp)
    s = np.where(np.arange(N) < N // 2, 1, -1)
    rowsum = A.astype(np.int64).sum(axis=1)
    np.testing.assert_array_equal(C, rowsum[:, None] * s[None, :])
    assert (C[: M // 2, : N // 2] == -128 * K).all()


# -- dX (catches: contraction over the wrong index, layout of the shared W) --------

@pytest.mark.parametrize("M,N,K,seed", [(1, 4, 16, 1), (9, 12, 20, 2), (27, 64, 96, 3), (5, 200, 8, 4)])
def test_dx_brute_force(M, N, K, seed):
    dC = synth.uniform_int8(seed, 2, M, N)
    codes = synth.random_codes(seed, N, K, 3)
    want = dC.astype(np.int64) @ lut_decode(codes).astype(np.int64)     # [M][N] x [N][K]
    np.testing.assert_array_equal(oracle.dx(dC, synth.store_codes(codes), K), want)


def test_dx_hand():
    # W (K=4 x N=2): n=0 codes 1,2,0,3 -> w(.,0) = +1,-1,0,0 ; n=1 all +1
    Wp = np.array([[0xC9], [0x55]], dtype=np.uint8)
    dC = np.array([[10, -3]], dtype=np.int8)
    # dX[k] = 10*w(k,0) - 3*w(k,1) = [10-3, -10-3, -3, -3]
    assert oracle.dx(dC, Wp, 4).tolist() == [[7, -13, -3, -3]]


def test_dx_is_forward_on_transposed_weights():
    M, N, K = 6, 24, 40
    dC = synth.uniform_int8(8, 2, M, N)
    codes = synth.random_codes(8, N, K, 4)               # [N][K]
    WpT = oracle.pack(np.ascontiguousarray(codes.T))     # codes along N, rows k
    np.testing.assert_array_equal(oracle.dx(dC, synth.store_codes(codes), K),
                                  oracle.fwd(dC, WpT))


# -- dW ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 1), (27, 16, 12, 2), (300, 33, 17, 3), (1782, 5, 7, 4)])
def test_dw_brute_force(M, N, K, seed):
    A = synth.uniform_int8(seed, 0, M, K)
    dC = synth.uniform_int8(seed, 2, M, N)
    want = A.astype(np.int64).T @ dC.astype(np.int64)
    np.testing.assert_array_equal(oracle.dw(A, dC, threads=4), want)


def test_dw_hand():
    A = np.array([[1, -2], [3, 4], [-5, 6]], dtype=np.int8)      # M=3, K=2
    dC = np.array([[7], [-1], [2]], dtype=np.int8)               # M=3, N=1
    # dW[0] = 1*7 + 3*(-1) + (-5)*2 = -6 ; dW[1] = -2*7 + 4*(-1) + 6*2 = -6
    assert oracle.dw(A, dC).tolist() == [[-6], [-6]]


def test_dw_int32_extremes_at_bound():
    M = read_kv("bounds.txt")["dw_max_contraction"]
    assert M == (2**31 - 1) // (128 * 128)
    A = np.full((M, 1), -128, dtype=np.int8)
    dC = np.empty((M, 2), dtype=np.int8)
    dC[:, 0] = -128
    dC[:, 1] = 127
    dW, r = oracle.dw(A, dC, return_overflows=True)
    assert r == 0
    assert dW.tolist() == [[2147467264, -2130690176]]


def test_dw_overflow_detected_past_bound():
    M = read_kv("bounds.txt")["dw_max_contraction"] + 1
    A = np.full((M, 1), -128, dtype=np.int8)
    dC = np.full((M, 1), -128, dtype=np.int8)
    _, r = oracle.dw(A, dC, allow_overflow=True, return_overflows=True)
    assert r == 1


# -- threading does not change the result ---------------------------------------

def test_thread_count_invariance():
    A, Wp = synth.fwd_inputs(21, 37, 19, 64, 4)
    base = oracle.fwd(A, Wp, threads=1)
    for t in (2, 5, 64):
        np.testing.assert_array_equal(oracle.fwd(A, Wp, threads=t), base)
    dC = synth.uniform_int8(21, 2, 37, 19)
    np.testing.assert_array_equal(oracle.dw(A, dC, threads=1), oracle.dw(A, dC, threads=7))
    np.testing.assert_array_equal(oracle.dx(dC, Wp, 64, threads=1), oracle.dx(dC, Wp, 64, threads=6))


def test_negative_overflow_detected():
    # below INT32_MIN: fwd with -128 x (+1) at K = 2^24 + 4, and dW with
    # -128 x 127 summed over 132105 rows (-16256 * 132105 = -2147498880)
    K = (1 << 24) + 4
    A = np.full((1, K), -128, dtype=np.int8)
    Wp = np.full((1, K // 4), 0x55, dtype=np.uint8)
    _, r = oracle.fwd(A, Wp, allow_overflow=True, return_overflows=True)
    assert r == 1
    M = 132105
    A = np.full((M, 1), -128, dtype=np.int8)
    dC = np.full((M, 1), 127, dtype=np.int8)
    dW, r = oracle.dw(A, dC, allow_overflow=True, return_overflows=True)
    assert r == 1
    assert int(dW[0, 0]) == -2147498880 + 2**32


# ---------------------------------------------------------------------------
# scaled outputs (the dequantization step after the integer product)
# ---------------------------------------------------------------------------

def test_bf16_rounding_hand_values():
    # catches: truncation instead of rounding, ties rounded up instead of to
    # even, overflow not going to inf, sign or NaN handling
    x = np.array([1.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -8 + 2 ** -20, 1 + 2 ** -8 - 2 ** -20,
                  -(1 + 3 * 2 ** -8), 3.3895313892515355e38, 3.4028234663852886e38, np.inf, -np.inf,
                  0.0, -0.0, 2.0 ** -133, 2.0 ** -134, 2.0 ** -134 + 2.0 ** -140], dtype=np.float32)
    want = [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0x3F80, 0xBF82, 0x7F7F, 0x7F80, 0x7F80, 0xFF80,
            0x0000, 0x8000, 0x0001, 0x0000, 0x0001]
    assert [int(v) for v in oracle.bf16_nearest_even(x)] == want
    nan = oracle.bf16_nearest_even(np.array([np.nan, -np.nan], dtype=np.float32))
    assert all((int(v) & 0x7F80) == 0x7F80 and (int(v) & 0x7F) != 0 and (int(v) & 0x40) for v in nan)


def test_bf16_rounding_matches_a_library():
    # catches: any rounding mistake at all -- torch's float32 -> bfloat16 cast
    # rounds to nearest even (NaN payloads excepted, checked above)
    torch = pytest.importorskip("torch")
    u = synth.splitmix64(11, 7, 1 << 20)
    bits = (u >> np.uint64(32)).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(oracle.bf16_nearest_even(x), want)


def test_scaled_f32_within_three_roundings_of_exact():
    # catches: a dropped or swapped scale, a wrong row/column orientation, a
    # product in lower precision -- the single-precision result must sit
    # within three half-ulp roundings of the exact real product
    R, C = 300, 272
    acc = (synth.splitmix64(5, 9, R * C) >> np.uint64(33)).astype(np.int64)
    acc = (acc - (1 << 30)).astype(np.int32).reshape(R, C)
    rs = synth.positive_scales(5, synth.STREAM_ROW_SCALE, R)
    cs = synth.positive_scales(5, synth.STREAM_COL_SCALE, C)
    exact = acc.astype(np.float64) * rs.astype(np.float64)[:, None] * cs.astype(np.float64)[None, :]
    y = oracle.scale_output(acc, rs, cs, "f32").astype(np.float64)
    assert np.all(np.abs(y - exact) <= 3 * 2.0 ** -24 * np.abs(exact))
    ys = oracle.scale_output(acc, rs, np.float32(synth.W_SCALE), "f32").astype(np.float64)
    exact_s = acc.astype(np.float64) * rs.astype(np.float64)[:, None] * np.float64(np.float32(synth.W_SCALE))
    assert np.all(np.abs(ys - exact_s) <= 3 * 2.0 ** -24 * np.abs(exact_s))
    # bf16 is within half a bf16 ulp (2^-8 of the value at most) of the f32 result
    yb = oracle.bf16_value(oracle.scale_output(acc, rs, cs, "bf16"))
    assert np.all(np.abs(yb - y) <= 2.0 ** -8 * np.abs(y))


def test_scaled_orientation_exact_case():
    # catches: row scales applied to columns (or the reverse); with powers of
    # two and small integers every value is exact
    acc = np.array([[1, 2, 3], [4, 5, 6]], dtype=np.int32)
    rs = np.array([0.5, 4.0], dtype=np.float32)
    cs = np.array([1.0, 0.25, 8.0], dtype=np.float32)
    want = np.array([[0.5, 0.25, 12.0], [16.0, 5.0, 192.0]], dtype=np.float32)
    np.testing.assert_array_equal(oracle.scale_output(acc, rs, cs, "f32"), want)
    np.testing.assert_array_equal(oracle.scale_output(acc, rs, np.float32(2.0), "f32"),
                                  acc * rs[:, None] * 2)
    # int32 -> float32 rounds to nearest even above 2^24
    big = np.array([[2 ** 24 + 1, 2 ** 24 + 3, -(2 ** 31)]], dtype=np.int32)
    got = oracle.scale_output(big, np.ones(1, np.float32), np.float32(1.0), "f32")
    np.testing.assert_array_equal(got, np.array([[2.0 ** 24, 2.0 ** 24 + 4, -2.0 ** 31]], np.float32))


# Exact-value pins of the two floating-point readings.  Expected values come
# from tests/exact_f32.py, an exact rational model of binary32 round-to-
# nearest-even, not from numpy's float32 arithmetic.  Each case was chosen
# (by a search with that model) so that the reading taken and a plausible
# alternative give different bits: a mistake in the order or kind of the
# steps fails here, where the error-bound pins above cannot tell.
#   scaled output:  RN(RN(acc * rs) * cs)      not  RN(acc * RN(rs * cs))
#   quantizer:      s = RN(max / 127)          not  RN(max * RN(1 / 127))
#                   q = rint(RN(x / s))        not  rint(RN(x * RN(1 / s)))
# ---------------------------------------------------------------------------

SCALE_ORDER_CASES = [(-124, 0x3DC059A7, 0x3D1C650C), (107, 0x3DC3078A, 0x3DBDC37C),
                     (85, 0x3DAB91B9, 0x3D641AF9)]          # (acc, row scale bits, column scale bits)
SCALE_DIVISION_CASES = [0x428E86F4, 0x424B1A5C, 0x429BE8FB]   # max |x| bits
VALUE_DIVISION_CASES = [(0x42C4A784, 0x419DF160), (0x42681D30, 0x419062C9),
                        (0x42B818E2, 0x412826DB), (0x429CF288, 0x4250D9EC)]   # (max |x| bits, x bits)


def _bits(a):
    return np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)


def test_exact_model_matches_ieee_on_hand_values():
    # the model itself, on values whose binary32 rounding is known by hand
    R = X.rn32
    assert R(Fraction(1, 3)) == Fraction(11184811, 2 ** 25)          # 0x3EAAAAAB
    assert R(Fraction(1) + Fraction(1, 2 ** 24)) == 1                   # tie -> even (1.0)
    assert R(Fraction(1) + Fraction(3, 2 ** 24)) == 1 + Fraction(2, 2 ** 23)   # tie -> even (up)
    assert R(Fraction(2 ** 24 + 1)) == 2 ** 24 and R(Fraction(2 ** 24 + 3)) == 2 ** 24 + 4
    assert R(Fraction(3, 2 ** 150)) == Fraction(2, 2 ** 149)             # subnormal tie -> even
    assert X.bits32(R(Fraction(1, 127))) == 0x3C010204


def test_scaled_output_order_exact_cases():
    for acc, rb, cb in SCALE_ORDER_CASES:
        rs, cs = X.f32_of_bits(rb), X.f32_of_bits(cb)
        want = X.rn32(X.rn32(acc * X.exact(rs)) * X.exact(cs))
        other = X.rn32(acc * X.rn32(X.exact(rs) * X.exact(cs)))
        assert want != other, "the case must separate the two orders"
        a = np.array([[acc]], dtype=np.int32)
        got = oracle.scale_output(a, np.array([rs]), np.array([cs]), "f32")
        assert int(_bits(got)[0, 0]) == X.bits32(want), (acc, hex(rb), hex(cb))
        got_s = oracle.scale_output(a, np.array([rs]), cs, "f32")       # one scale for every column
        assert int(_bits(got_s)[0, 0]) == X.bits32(want)


def test_scaled_output_every_element_exact():
    # every element of a random case against the exact model, acc up to 2^30
    # (so the int32 -> float conversion rounds too)
    R, C = 12, 10
    acc = ((synth.splitmix64(21, 9, R * C) >> np.uint64(33)).astype(np.int64) - (1 << 30)).astype(np.int32)
    acc = acc.reshape(R, C)
    rs = synth.positive_scales(21, synth.STREAM_ROW_SCALE, R)
    cs = synth.positive_scales(21, synth.STREAM_COL_SCALE, C)
    got = _bits(oracle.scale_output(acc, rs, cs, "f32"))
    for r in range(R):
        for c in range(C):
            y = X.rn32(X.rn32(X.rn32(Fraction(int(acc[r, c]))) * X.exact(rs[r])) * X.exact(cs[c]))
            assert int(got[r, c]) == X.bits32(y), (r, c)


def test_quantize_scale_is_a_division_exact_cases():
    inv127 = X.rn32(Fraction(1, 127))
    for mb in SCALE_DIVISION_CASES:
        m = X.f32_of_bits(mb)
        s = X.rn32(X.exact(m) / 127)
        assert s != X.rn32(X.exact(m) * inv127), "the case must separate the two readings"
        x = np.array([[m, -m / np.float32(3), np.float32(0.25)]], dtype=np.float32)
        for axis, xin in (("rows", x), ("cols", np.ascontiguousarray(x.T))):
            _, sc = oracle.quantize(xin, "f32", axis)
            assert int(_bits(sc)[0]) == X.bits32(s), (axis, hex(mb))


def test_quantize_value_is_a_division_exact_cases():
    for mb, xb in VALUE_DIVISION_CASES:
        m, x = X.f32_of_bits(mb), X.f32_of_bits(xb)
        s = X.rn32(X.exact(m) / 127)
        q = X.round_half_even(X.rn32(X.exact(x) / s))
        other = X.round_half_even(X.rn32(X.exact(x) * X.rn32(1 / s)))
        assert q != other, "the case must separate the two readings"
        row = np.array([[m, x, -x]], dtype=np.float32)
        for axis, xin in (("rows", row), ("cols", np.ascontiguousarray(row.T))):
            qv, _ = oracle.quantize(xin, "f32", axis)
            qv = qv.reshape(-1)
            assert qv.tolist() == [127, q, -q], (axis, hex(mb), hex(xb))


def test_quantize_every_element_exact():
    # every element of random rows against the exact model of the rule
    x = synth.float_inputs(22, synth.STREAM_X, 6, 40, "f32")
    q, s = oracle.quantize(x, "f32", "rows")
    for r in range(x.shape[0]):
        m = max(abs(X.exact(v)) for v in x[r])
        sr = X.rn32(m / 127)
        assert int(_bits(s)[r]) == X.bits32(sr)
        for c in range(x.shape[1]):
            qq = max(-127, min(127, X.round_half_even(X.rn32(X.exact(x[r, c]) / sr))))
            assert int(q[r, c]) == qq, (r, c)


# ---------------------------------------------------------------------------
# packing the trainer's ternary weights (codes by sign) and the per-row /
# per-column int8 quantizer (symmetric absmax, IEEE single precision)
# ---------------------------------------------------------------------------

def test_pack_weights_hand_bytes():
    # row [+1, -1, 0, +1] -> codes 1, 2, 0, 1 -> 1 + (2 << 2) + (0 << 4) + (1 << 6) = 0x49;
    # signs only: [127, -128, 5, 0] -> codes 1, 2, 1, 0 -> 0x19
    Wt = np.array([[1, -1, 0, 1, 127, -128, 5, 0]], dtype=np.int8)
    assert oracle.pack_weights(Wt).tolist() == [[0x49, 0x19]]


def test_pack_weights_round_trip_through_the_page_decode():
    # decoding the packed ternary weights with the pages' table gives them back
    Wt = synth.ternary_int8(3, 37, 96)
    assert set(np.unique(Wt).tolist()) == {-1, 0, 1}
    np.testing.assert_array_equal(oracle.decode(oracle.pack_weights(Wt), 96), Wt)


def test_pack_weights_is_sign_of_any_int8():
    W = synth.uniform_int8(4, synth.STREAM_A, 19, 64)
    np.testing.assert_array_equal(oracle.decode(oracle.pack_weights(W), 64), np.sign(W).astype(np.int8))
    assert 3 not in oracle.unpack(oracle.pack_weights(W), 64)


def test_quantize_integer_row_with_max_127_is_identity():
    # max |x| = 127 gives s = 1 exactly, and integer values stay as they are
    x = np.array([[127, -127, 3, 0, -64, 1], [-127, 5, 0, 0, 2, 126]], dtype=np.float32)
    q, s = oracle.quantize(x, "f32", "rows")
    assert s.tolist() == [1.0, 1.0]
    np.testing.assert_array_equal(q, x.astype(np.int8))


def test_quantize_ties_round_to_even():
    x = np.array([[127, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 126.5]], dtype=np.float32)
    q, s = oracle.quantize(x, "f32", "rows")
    assert s.tolist() == [1.0]
    assert q.tolist() == [[127, 2, 4, -2, -4, 0, 0, 126]]


def test_quantize_power_of_two_scaling_is_exact():
    x = synth.float_inputs(5, synth.STREAM_X, 7, 33, "f32")
    q, s = oracle.quantize(x, "f32", "rows")
    for e in (-12, -1, 5):
        q2, s2 = oracle.quantize(x * np.float32(2.0 ** e), "f32", "rows")
        np.testing.assert_array_equal(q2, q)
        np.testing.assert_array_equal(s2, s * np.float32(2.0 ** e))


def test_quantize_zero_row_and_signs():
    x = np.zeros((3, 8), dtype=np.float32)
    x[1] = np.linspace(-3, 3, 8, dtype=np.float32)
    x[2, 3] = -0.0
    q, s = oracle.quantize(x, "f32", "rows")
    assert s[0] == 0 and s[2] == 0 and not q[0].any() and not q[2].any()
    qn, sn = oracle.quantize(-x, "f32", "rows")
    np.testing.assert_array_equal(qn, -q)
    np.testing.assert_array_equal(sn, s)


def test_quantize_error_within_half_a_step():
    # against float64: |q s - x| <= s / 2 plus the one rounding of x / s
    x = synth.float_inputs(6, synth.STREAM_X, 64, 300, "f32")
    q, s = oracle.quantize(x, "f32", "rows")
    err = np.abs(q.astype(np.float64) * s[:, None].astype(np.float64) - x.astype(np.float64))
    assert (err <= s[:, None].astype(np.float64) * (0.5 + 127 * 2.0 ** -23)).all()
    # the largest magnitude of each row maps to +-127
    i = np.abs(x).argmax(axis=1)
    assert (np.abs(q[np.arange(64), i]) == 127).all()
    # s is max|x| / 127 to within one rounding
    assert np.allclose(s.astype(np.float64) * 127, np.abs(x).max(axis=1), rtol=2.0 ** -23, atol=0)


def test_quantize_columns_are_rows_of_the_transpose():
    x = synth.float_inputs(7, synth.STREAM_X, 45, 29, "f32")
    qc, sc = oracle.quantize(x, "f32", "cols")
    qr, sr = oracle.quantize(np.ascontiguousarray(x.T), "f32", "rows")
    np.testing.assert_array_equal(qc, qr.T)
    np.testing.assert_array_equal(sc, sr)


def test_quantize_bf16_input_widening():
    b = np.array([[0x3F80, 0xC000, 0x0000, 0x8000, 0x42FE]], dtype=np.uint16)   # 1, -2, 0, -0, 127
    assert oracle.as_float32(b, "bf16").tolist() == [[1.0, -2.0, 0.0, -0.0, 127.0]]
    q, s = oracle.quantize(b, "bf16", "rows")
    assert s.tolist() == [1.0] and q.tolist() == [[1, -2, 0, 0, 127]]
    xb = synth.float_inputs(8, synth.STREAM_X, 5, 40, "bf16")
    np.testing.assert_array_equal(oracle.quantize(xb, "bf16", "rows")[0],
                                  oracle.quantize(oracle.as_float32(xb, "bf16"), "f32", "rows")[0])
