"""Pins for the oracle GEMM: C = fp16(sum_k A[i,k] B[k,j]), fp64 ascending-k sum, one rounding.

Definition: phobos "03: Matrix multiplication" (docstring, kernel and the paragraph after
it): fp16 operands, fp32 accumulator, one narrowing to fp16 on the store.  The oracle sums
in fp64, which is exact for the inputs here whenever the span of the products fits 53 bits.

Pins (none re-computes the oracle's own formula the same way):
  * exact big-integer brute force on tiny shapes, with subnormals;
  * numpy's float64 BLAS product on inputs whose sums are exact in fp64 (any order);
  * closed forms: identity, zero, one-hots on the last row/column, all-ones sums and the
    round-half-even ties they produce (K = 2051, 4093, 4095);
  * invariants: power-of-two scaling, transposition, padding left untouched, K = 0.
"""
import numpy as np
import pytest

import oracle
from exact_fp16 import gemm_exact, round_scaled_to_f16
from synthetic_inputs import operands


def f16(x):
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def as_f64(h):
    return np.asarray(h, dtype=np.uint16).view(np.float16).astype(np.float64)


def random_f16(rng, shape, lo_exp=-24, hi_exp=3):
    """Random finite fp16 patterns with magnitudes spread over 2^lo_exp .. 2^hi_exp."""
    mag = np.exp2(rng.uniform(lo_exp, hi_exp, shape))
    sgn = rng.choice([-1.0, 1.0], shape)
    return f16(mag * sgn)


@pytest.mark.parametrize("M,N,K,seed", [(1, 1, 1, 0), (3, 5, 7, 1), (16, 16, 16, 2),
                                        (9, 13, 64, 3), (32, 24, 40, 4)])
def test_exact_bruteforce_narrow_span(M, N, K, seed):
    """Values in [2^-8, 1): every fp64 partial sum is exact, so bit-exact to exact rounding."""
    rng = np.random.default_rng(seed)
    A = random_f16(rng, (M, K), -8, 0)
    B = random_f16(rng, (K, N), -8, 0)
    assert np.array_equal(oracle.gemm(A, B), gemm_exact(A, B))


@pytest.mark.parametrize("seed", range(4))
def test_exact_bruteforce_with_subnormals(seed):
    """Full fp16 range incl. subnormals: fp64 sums may round, so allow 1 ulp, rarely."""
    rng = np.random.default_rng(100 + seed)
    M, N, K = 12, 10, 48
    A = random_f16(rng, (M, K), -24, 7)
    B = random_f16(rng, (K, N), -24, 7)
    got = oracle.gemm(A, B).astype(np.int32)
    want = gemm_exact(A, B).astype(np.int32)
    diff = got != want
    # where they differ, they must be neighbours (same sign, adjacent patterns)
    assert np.all(np.abs(got[diff] - want[diff]) <= 1)
    assert diff.sum() <= 2


def test_matches_numpy_blas_when_sums_are_exact():
    """Grid inputs (multiples of 2^-11 in [-0.5, 0.5)) have exact fp64 sums in any order."""
    A, B = operands(96, 80, 200, "u(-0.5,0.5)", 11)
    want = f16(as_f64(A) @ as_f64(B))
    assert np.array_equal(oracle.gemm(A, B), want)
    A, B = operands(64, 48, 130, "u(0,1)", 12)
    want = f16(as_f64(A) @ as_f64(B))
    assert np.array_equal(oracle.gemm(A, B), want)


def test_identity_and_zero():
    rng = np.random.default_rng(5)
    B = random_f16(rng, (37, 29), -20, 10)
    eye = f16(np.eye(37))
    assert np.array_equal(oracle.gemm(eye, B), B)
    Z = np.zeros((11, 37), dtype=np.uint16)
    assert np.array_equal(oracle.gemm(Z, B), np.zeros((11, 29), dtype=np.uint16))


def test_one_hot_selects_last_row_and_column():
    rng = np.random.default_rng(6)
    M, N, K = 7, 9, 33
    B = random_f16(rng, (K, N), -10, 4)
    A = np.zeros((M, K), dtype=np.uint16)
    A[:, K - 1] = f16(1.0)
    C = oracle.gemm(A, B)
    assert np.array_equal(C, np.broadcast_to(B[K - 1], (M, N)))
    # one-hot in the last row of A picks out a row of B only in the last row of C
    A = np.zeros((M, K), dtype=np.uint16)
    A[M - 1, 3] = f16(1.0)
    C = oracle.gemm(A, B)
    assert np.array_equal(C[M - 1], B[3]) and not C[:M - 1].any()
    # one-hot in the last column of B
    Ar = random_f16(rng, (M, K), -10, 4)
    Bo = np.zeros((K, N), dtype=np.uint16)
    Bo[K - 1, N - 1] = f16(1.0)
    C = oracle.gemm(Ar, Bo)
    assert np.array_equal(C[:, N - 1], Ar[:, K - 1]) and not C[:, :N - 1].any()


@pytest.mark.parametrize("K,want", [(1, 1.0), (1000, 1000.0), (2048, 2048.0), (2049, 2048.0),
                                    (2051, 2052.0), (4093, 4092.0), (4095, 4096.0)])
def test_all_ones_round_half_even(K, want):
    """sum of K ones = K; above 2048 fp16 spacing is 2, so odd K are ties to the even pattern."""
    A = f16(np.ones((2, K)))
    B = f16(np.ones((K, 3)))
    C = oracle.gemm(A, B)
    assert np.all(C == f16(want))
    assert round_scaled_to_f16(K, 0) == int(f16(want))


def test_power_of_two_scaling():
    A, B = operands(40, 30, 64, "u(-0.5,0.5)", 21)
    C = oracle.gemm(A, B)
    for e in (-2, 3):
        As = f16(as_f64(A) * 2.0 ** e)
        Cs = oracle.gemm(As, B)
        ok = np.abs(as_f64(C)) >= 2.0 ** -10     # normal before and after scaling
        assert np.array_equal(as_f64(Cs)[ok], as_f64(C)[ok] * 2.0 ** e)


def test_transpose_invariant():
    rng = np.random.default_rng(8)
    A = random_f16(rng, (23, 41), -12, 2)
    B = random_f16(rng, (41, 17), -12, 2)
    C = oracle.gemm(A, B)
    Ct = oracle.gemm(np.ascontiguousarray(B.T), np.ascontiguousarray(A.T))
    assert np.array_equal(Ct.T, C)


def test_leading_dimensions_and_padding_untouched():
    A, B = operands(33, 21, 45, "n(0,0.1)", 9)
    C = oracle.gemm(A, B)
    Ap = np.full((33, 50), 0x7E00, dtype=np.uint16)   # NaN padding must never be read
    Ap[:, :45] = A
    Bp = np.full((45, 29), 0x7E00, dtype=np.uint16)
    Bp[:, :21] = B
    Cp = np.full((33, 25), 0xABCD, dtype=np.uint16)
    oracle.gemm(Ap, Bp, Cp, M=33, N=21, K=45)
    assert np.array_equal(Cp[:, :21], C)
    assert np.all(Cp[:, 21:] == 0xABCD)


def test_k_zero_gives_positive_zero_and_empty_is_noop():
    A = np.zeros((4, 0), dtype=np.uint16)
    B = np.zeros((0, 5), dtype=np.uint16)
    C = np.full((4, 5), 0x1234, dtype=np.uint16)
    oracle.gemm(A, B, C, M=4, N=5, K=0)
    assert np.all(C == 0x0000)
    C = np.full((4, 5), 0x1234, dtype=np.uint16)
    oracle.gemm(np.zeros((0, 3), np.uint16), np.zeros((3, 5), np.uint16), C, M=0, N=5, K=3)
    assert np.all(C == 0x1234)


def test_sampled_matches_full():
    A, B = operands(70, 90, 130, "n(0,0.1)", 4)
    C = oracle.gemm(A, B)
    rng = np.random.default_rng(3)
    r = rng.integers(0, 70, 500)
    c = rng.integers(0, 90, 500)
    got, s = oracle.gemm_sampled(A, B, r, c, want_f64=True)
    assert np.array_equal(got, C[r, c])
    assert np.array_equal(f16(s), got)


# ---------------------------------------------------------------------------------------
# The blocked form (64 x 256 blocks of C, k outermost inside a block) on shapes that span
# several blocks and end in partial ones.
# ---------------------------------------------------------------------------------------
def test_multi_block_matches_numpy_blas_when_sums_are_exact():
    """Across block edges (rows 64, 128, columns 256, 512 and ragged last blocks) the result
    is the one numpy's float64 product gives when every sum is exact in fp64."""
    A, B = operands(150, 600, 300, "u(-0.5,0.5)", 31)
    assert np.array_equal(oracle.gemm(A, B), f16(as_f64(A) @ as_f64(B)))
    A, B = operands(65, 257, 129, "u(0,1)", 32)
    assert np.array_equal(oracle.gemm(A, B), f16(as_f64(A) @ as_f64(B)))


def test_multi_block_identity_and_one_hot():
    rng = np.random.default_rng(33)
    B = random_f16(rng, (300, 530), -20, 10)
    assert np.array_equal(oracle.gemm(f16(np.eye(300)), B), B)
    A = np.zeros((130, 300), dtype=np.uint16)
    A[:, 299] = f16(1.0)
    assert np.array_equal(oracle.gemm(A, B), np.broadcast_to(B[299], (130, 530)))


@pytest.mark.parametrize("M,N,K", [(130, 520, 77), (65, 257, 300), (1, 700, 40), (200, 3, 90),
                                   (64, 256, 5), (129, 513, 1)])
def test_blocked_equals_one_dot_per_element(M, N, K):
    """Both forms add each element's products in ascending k, so they agree bit for bit --
    with subnormals, infinities and NaNs among the operands too.  The sign of a NaN result is
    not part of the definition (the two loops may hand the adder its operands in either
    order, and x86 keeps the first NaN operand's sign), so NaNs compare as one value."""
    rng = np.random.default_rng(M * 1000 + N + K)
    A = random_f16(rng, (M, K), -24, 8)
    B = random_f16(rng, (K, N), -24, 8)
    for X, count in ((A, 3), (B, 3)):
        r = rng.integers(0, X.shape[0], count)
        c = rng.integers(0, X.shape[1], count)
        X[r, c] = rng.choice([0x7C00, 0xFC00, 0x7E00], count)
    def canon(h):
        h = h.copy()
        h[((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)] = 0x7E00
        return h

    blocked, plain = oracle.gemm(A, B), oracle.gemm(A, B, plain=True)
    assert np.array_equal(canon(blocked), canon(plain))
