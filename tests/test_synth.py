"""The seeded input generator: published test vector, determinism, value maps."""
import numpy as np

from ternary_weight_int8_amd import synth


def test_splitmix64_published_vector():
    # seed 0, stream 0 gives a start state of 0, so the draws are those of a
    # plain SplitMix64 started at 0; its first output is the well-known
    # 0xE220A8397B1DCDAF.
    assert synth.stream_base(0, 0) == 0
    u = synth.splitmix64(0, 0, 1)
    assert int(u[0]) == 0xE220A8397B1DCDAF


def test_counter_form_equals_sequential_form():
    base = synth.stream_base(1234, 1)
    u = synth.splitmix64(1234, 1, 6)
    s = base
    for i in range(6):
        s = (s + 0x9E3779B97F4A7C15) & (2**64 - 1)
        z = s
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & (2**64 - 1)
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & (2**64 - 1)
        z ^= z >> 31
        assert int(u[i]) == z


def test_offsets_slice_the_same_stream():
    full = synth.splitmix64(9, 2, 100)
    np.testing.assert_array_equal(synth.splitmix64(9, 2, 30, offset=50), full[50:80])


def test_streams_and_seeds_differ():
    a = synth.splitmix64(5, 0, 64)
    assert not np.array_equal(a, synth.splitmix64(5, 1, 64))
    assert not np.array_equal(a, synth.splitmix64(6, 0, 64))


def test_int8_value_map():
    A = synth.uniform_int8(1, 0, 256, 1024)
    assert A.dtype == np.int8
    assert A.min() == -128 and A.max() == 127
    assert abs(A.astype(np.float64).mean() + 0.5) < 0.5
    u = synth.splitmix64(1, 0, 8)
    assert [int(x) for x in A.reshape(-1)[:8].view(np.uint8)] == [int(x) >> 56 for x in u]


def test_code_alphabets():
    c4 = synth.random_codes(3, 200, 1000, 4)
    c3 = synth.random_codes(3, 200, 1000, 3)
    n = c4.size
    for c in range(4):
        assert abs((c4 == c).sum() / n - 0.25) < 0.01
    assert (c3 <= 2).all()
    for c in range(3):
        assert abs((c3 == c).sum() / n - 1 / 3) < 0.01


def test_determinism():
    a1, w1 = synth.fwd_inputs(42, 33, 17, 64, 3)
    a2, w2 = synth.fwd_inputs(42, 33, 17, 64, 3)
    np.testing.assert_array_equal(a1, a2)
    np.testing.assert_array_equal(w1, w2)
    assert w1.shape == (17, 16)


def test_store_codes_bit_placement():
    codes = np.array([[1, 2, 0, 3, 2, 2, 2, 2]], dtype=np.uint8)
    assert synth.store_codes(codes).tolist() == [[0xC9, 0xAA]]


def test_extreme_inputs_structure():
    A, Wp = synth.extreme_inputs(1, 8, 6, 16)
    assert (A[:4] == -128).all()
    assert not (A[4:] == -128).all()
    assert (Wp[:3] == 0x55).all() and (Wp[3:] == 0xAA).all()
    # the uniform rows are the stream's values at their own storage indices
    u = synth.splitmix64(1, 0, 4 * 16, offset=4 * 16)
    np.testing.assert_array_equal(A[4:].reshape(-1).view(np.uint8),
                                  (u >> np.uint64(56)).astype(np.uint8))


def test_float_inputs_ranges_and_determinism():
    x = synth.float_inputs(1, synth.STREAM_X, 50, 64, "f32")
    assert x.dtype == np.float32 and np.isfinite(x).all()
    nz = np.abs(x[x != 0])
    assert nz.min() >= 2.0 ** -8 and nz.max() < 2.0 ** 4
    assert (x == 0).sum() > 0
    np.testing.assert_array_equal(x, synth.float_inputs(1, synth.STREAM_X, 50, 64, "f32"))
    b = synth.float_inputs(1, synth.STREAM_X, 50, 64, "bf16")
    assert b.dtype == np.uint16
    assert (((b >> 7) & 0xFF)[b & 0x7FFF != 0] >= 127 - 8).all()


def test_ternary_int8_values():
    w = synth.ternary_int8(2, 30, 200)
    assert w.dtype == np.int8 and set(np.unique(w).tolist()) == {-1, 0, 1}
    counts = np.bincount((w.astype(np.int16) + 1).ravel())
    assert counts.min() > 0.3 * w.size / 3
