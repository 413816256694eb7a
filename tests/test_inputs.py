"""Pins for the seeded operand generator (no GEMM arithmetic lives there)."""
import numpy as np

from synthetic_inputs import operands, splitmix64, stream


def test_splitmix64_published_vector():
    # First outputs of SplitMix64 seeded with 1234567 (the generator's reference test vector).
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423,
            4593380528125082431, 16408922859458223821]
    assert splitmix64(1234567, 0, 5).tolist() == want


def test_counter_based_chunks_agree():
    whole = stream("n(0,0.1)", 4, 0, 5000)
    parts = np.concatenate([stream("n(0,0.1)", 4, a, 1000) for a in range(0, 5000, 1000)])
    assert np.array_equal(whole, parts)
    odd = stream("n(0,0.1)", 4, 1001, 7)
    assert np.array_equal(odd, whole[1001:1008])


def test_uniform_grids_exact_and_in_range():
    A, B = operands(300, 200, 100, "u(-0.5,0.5)", 0)
    v = A.view(np.float16).astype(np.float64)
    assert v.min() >= -0.5 and v.max() < 0.5
    assert np.all(v * 2048 == np.round(v * 2048))
    A, B = operands(300, 200, 100, "u(0,1)", 1)
    v = B.view(np.float16).astype(np.float64)
    assert v.min() >= 0 and v.max() < 1
    assert np.all(v * 2048 == np.round(v * 2048))


def test_normal_moments():
    A, _ = operands(1000, 1, 1000, "n(0,0.1)", 4)
    v = A.view(np.float16).astype(np.float64)
    assert abs(v.mean()) < 2e-3 and abs(v.std() - 0.1) < 2e-3


def test_b_continues_the_stream():
    A, B = operands(3, 4, 5, "u(0,1)", 1)
    s = stream("u(0,1)", 1, 0, 3 * 5 + 5 * 4)
    assert np.array_equal(A.ravel(), s[:15]) and np.array_equal(B.ravel(), s[15:])


def test_low_activity_distributions():
    A, B = operands(64, 32, 48, "zeros", 3)
    assert not A.any() and not B.any()
    A, B = operands(500, 300, 400, "s(1/64)", 3)
    v = np.concatenate([A.ravel(), B.ravel()]).view(np.float16).astype(np.float64)
    assert set(np.unique(v)) == {-1 / 64, 1 / 64}
    assert abs(np.mean(v > 0) - 0.5) < 0.01
    # the sign bit is the top bit of the same draws whose top 11 bits index the uniform grid
    # (top bit set: grid index >= 1024, a value >= 0; here the negative value)
    u = stream("u(-0.5,0.5)", 3, 0, 1000).view(np.float16)
    s = stream("s(1/64)", 3, 0, 1000).view(np.float16)
    assert np.array_equal(s < 0, u >= 0)
