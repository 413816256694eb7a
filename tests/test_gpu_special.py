"""IEEE special values through the GPU path, against the oracle bit for bit.

The pages say nothing about overflow, NaN, infinities, subnormals or the sign of zero; the
reading is IEEE propagation (fp16 x fp16 products are exact in fp32, sums in fp32, one
round-to-nearest-even narrowing, which overflows to infinity at |s| >= 65520).  Every case
below is built so that all partial sums are exact in fp32, so the one correct result is the
oracle's, in every k order: the comparison is bit for bit, NaN meeting NaN (any payload).
"""
import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import from_dev, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def h(x):
    return np.float16(x).view(np.uint16)


INF, NINF, NAN, NZERO = 0x7C00, 0xFC00, 0x7E00, 0x8000


def assert_same_bits(gpu, want, what):
    gn = (gpu & 0x7C00) == 0x7C00
    gn &= (gpu & 0x03FF) != 0                   # NaN: exponent all ones, mantissa non-zero
    wn = ((want & 0x7C00) == 0x7C00) & ((want & 0x03FF) != 0)
    assert np.array_equal(gn, wn), f"{what}: NaN positions differ"
    assert np.array_equal(np.where(wn, 0, gpu), np.where(wn, 0, want)), f"{what}: bits differ"


def run_all_ways(A, B, what):
    """Row-major DMA path, forced generic path, B given column-major, and the large tiles'
    own kernels: the 256 x 256 x 64 tile (16x16x32 MFMAs in its five-slot schedule, also
    persistent and split in two along k), the ping-pong tile and the four-stage 256 x 256 x 32
    tile (32x32x16 MFMAs)."""
    M, K = A.shape
    N = B.shape[1]
    want = oracle.gemm(A, B)
    Ad, Bd = to_dev(A), to_dev(B)
    assert_same_bits(from_dev(g.matmul(Ad, Bd)), want, what + " dma")
    assert_same_bits(from_dev(g.matmul(Ad, Bd, force_generic=1)), want, what + " generic")
    Bt = to_dev(np.ascontiguousarray(B.T)).t()
    assert_same_bits(from_dev(g.matmul(Ad, Bt)), want, what + " B column-major")
    for t in (g.TILE_256x256x64, g.TILE_256x256x32_PP, g.TILE_256x256x32):
        assert_same_bits(from_dev(g.matmul(Ad, Bd, tile=t)), want, f"{what} tile {t}")
    t1 = g.TILE_256x256x64
    assert_same_bits(from_dev(g.matmul(Ad, Bd, tile=t1, persistent=g.PERSISTENT_ON)), want,
                     what + " persistent")
    # two slices when K > 128; the slices' fp32 sums are exact here too, so their sum is
    assert_same_bits(from_dev(g.matmul(Ad, Bd, tile=t1, split_k=2)), want, what + " split")
    return want


def test_overflow_to_signed_infinity():
    """Narrowing overflows to infinity from |s| >= 65520 on (65520 itself is the tie between
    65504 and 2^16, and ties go to the even one, 2^16 = inf)."""
    M, N, K = 200, 130, 96
    A = np.full((M, K), h(1.0), np.uint16)
    B = np.full((K, N), h(1.0), np.uint16)
    B[:, 9] = h(256.0)
    B[:, 10] = h(32.0)
    A[5:12] = 0
    A[5] = h(256.0)                          # column 9: 96 * 65536: +inf
    A[6] = h(-256.0)                         # -inf
    A[7, 0], A[7, 1] = h(255.0), h(1.0)      # column 9: 65280 + 256 = 65536: +inf
    A[8, 0] = h(255.0)                       # column 9: 65280, finite
    A[9, 0] = h(2047.0)                      # column 10: 65504, the largest finite value
    A[10, 0], A[10, 1] = h(2047.0), h(0.25)  # column 10: 65512 rounds down to 65504
    A[11, 0], A[11, 1] = h(2047.0), h(0.5)   # column 10: 65520, the tie: +inf
    want = run_all_ways(A, B, "overflow")
    assert (want[5, 9], want[6, 9], want[7, 9]) == (INF, NINF, INF)
    assert want[8, 9] == h(65280.0)
    assert want[9, 10] == h(65504.0) and want[10, 10] == h(65504.0) and want[11, 10] == INF


def test_nan_and_infinity_propagation():
    M, N, K = 160, 140, 70
    A = np.full((M, K), h(0.5), np.uint16)
    B = np.full((K, N), h(0.25), np.uint16)
    A[3, 5] = NAN                  # row 3 becomes NaN
    B[7, 2] = NAN                  # column 2 becomes NaN
    A[10, 0] = INF                 # inf x 0 = NaN where B[0][j] == 0, inf where B[0][j] > 0
    B[0, :] = 0
    B[0, 1] = h(1.0)
    A[20, 1] = INF                 # inf - inf = NaN where B[1][j] < 0 and B[2][j] > 0 ...
    A[20, 2] = INF
    B[1, 40:] = h(-1.0)
    want = run_all_ways(A, B, "nan/inf")
    nan = lambda v: (v & 0x7C00) == 0x7C00 and (v & 0x3FF) != 0
    assert all(nan(v) for v in want[3]) and all(nan(v) for v in want[:, 2])
    assert want[10, 1] == INF and nan(want[10, 0])
    assert nan(want[20, 50]) and want[20, 30] == INF


def test_subnormal_operands_and_results():
    """Subnormal fp16 inputs are used at their value (not flushed), products below fp16's
    range survive in fp32, and results land in fp16's subnormal range when they are small."""
    M, N, K = 96, 80, 64
    rng = np.random.default_rng(5)
    # A: subnormals n * 2^-24 with n in 1..1023; B: small integers
    A = (rng.integers(1, 1024, (M, K))).astype(np.uint16)          # bit pattern = n: n * 2^-24
    B = np.array([h(float(v)) for v in rng.integers(-3, 4, K * N)], np.uint16).reshape(K, N)
    want = run_all_ways(A, B, "subnormal inputs")
    assert np.any((want & 0x7C00) == 0) and np.any(want != 0)
    # 2^-14 x 2^-14 = 2^-28 (zero in fp16, exact in fp32); 16 of them sum to 2^-24
    A2 = np.full((64, 16), h(2.0 ** -14), np.uint16)
    B2 = np.full((16, 64), h(2.0 ** -14), np.uint16)
    want2 = run_all_ways(A2, B2, "tiny products")
    assert np.all(want2 == 1)                                     # 2^-24: the least subnormal
    # 3 * 2^-26 = 0.75 * 2^-24 rounds to 2^-24; 2^-26 rounds to +0
    A3 = np.zeros((64, 16), np.uint16)
    A3[:, :3] = h(2.0 ** -13)
    A3[32:, 1:3] = 0
    B3 = np.full((16, 64), h(2.0 ** -13), np.uint16)
    want3 = run_all_ways(A3, B3, "rounding into the subnormal range")
    assert np.all(want3[:32] == 1) and np.all(want3[32:] == 0)


def test_signed_zero():
    """Sums start from +0: all-(-0) products, and exact cancellation, both give +0."""
    M, N, K = 64, 64, 32
    A = np.full((M, K), NZERO, np.uint16)
    B = np.full((K, N), h(1.0), np.uint16)
    assert np.all(run_all_ways(A, B, "-0 products") == 0)
    A = np.full((M, K), h(1.0), np.uint16)
    B = np.full((K, N), h(1.0), np.uint16)
    B[: K // 2] = h(-1.0)
    assert np.all(run_all_ways(A, B, "cancellation") == 0)


def test_special_values_across_split_k_slices():
    """K = 300 in two slices (k < 44 and k >= 44, each summed in fp32, then added): an
    infinity in each slice of opposite signs gives NaN, of the same sign infinity; a NaN in
    one slice wins; a slice sum beyond fp16's range with a finite total of the other slice
    still overflows on the one narrowing; values cancelling across slices give +0."""
    M, N, K = 70, 90, 300
    A = np.full((M, K), h(0.5), np.uint16)
    B = np.full((K, N), h(0.25), np.uint16)
    A[1, 3], A[1, 200] = INF, NINF           # row 1: +inf (slice 0) and -inf (slice 1): NaN
    A[2, 3], A[2, 200] = INF, INF            # row 2: +inf
    A[3, 250] = NAN                          # row 3: NaN from slice 1
    A[4, :] = h(2047.0)                      # row 4: 300 x 2047 x 0.25 = 153525: +inf
    A[5, :] = h(1.0)
    A[5, 44:] = h(-1.0)                      # row 5 with column 7 all ones: 44 - 256
    B[:, 7] = h(1.0)
    A[6, :44] = h(64.0)                      # row 6: 64 x 44 - 11.0 x 256, column 7: 0
    A[6, 44:] = h(-11.0)
    want = run_all_ways(A, B, "split slices")
    rc, info = g.gemm_f16f32_plan(M, N, K, 1 << 40, 2 << 40, 3 << 40, K, N, N,
                                  opts={"tile": g.TILE_256x256x64, "split_k": 2})
    assert rc == g.OK and info["splits"] == 2 and info["split_depth"] == 256
    nan = lambda v: (v & 0x7C00) == 0x7C00 and (v & 0x3FF) != 0
    assert all(nan(v) for v in want[1]) and np.all(want[2] == INF)
    assert all(nan(v) for v in want[3]) and np.all(want[4] == INF)
    assert want[5, 7] == h(44.0 - 256.0) and want[6, 7] == 0
