"""GPU parity of the strided entry point: every storage order of A, B and C.

The notebook's kernel takes a stride per axis of every matrix (stride_am, stride_ak,
stride_bk, stride_bn, cell In[8]); gemm_f16f32_strided accepts any row- or column-major
storage.  An operand's storage order changes only how its panels are staged, never the
values an MFMA receives or the order of the k-sum, so every layout must give the row-major
result bit for bit; that result is itself checked against the oracle.  Padding between the
rows (columns) of the stored matrices holds NaN, which would poison any sum that read it,
and C's padding holds a canary that must survive.
"""
import itertools

import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import (assert_within_tolerance, from_dev, output, padding_untouched, place,
                      to_dev)
from synthetic_inputs import operands

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LAYOUTS = list(itertools.product((False, True), repeat=3))  # (A col-major, B col-major, C col-major)


def call(Av, Bv, Cv, **opts):
    M, K = Av.shape
    N = Bv.shape[1]
    rc = g.gemm_f16f32_strided(M, N, K, Av.data_ptr(), Av.stride(0), Av.stride(1),
                               Bv.data_ptr(), Bv.stride(0), Bv.stride(1), Cv.data_ptr(),
                               Cv.stride(0), Cv.stride(1),
                               torch.cuda.current_stream().cuda_stream, opts or None)
    assert rc == g.OK, g.gemm_f16f32_strerror(rc)
    return from_dev(Cv)


def row_major_result(A, B, **opts):
    return from_dev(g.matmul(to_dev(A), to_dev(B), **opts))


SHAPES = [(512, 512, 512), (300, 264, 200), (1000, 600, 300), (257, 129, 65), (1, 1, 1),
          (64, 1, 1000), (1, 77, 33), (129, 65, 4093)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_every_layout_equals_row_major(M, N, K):
    A, B = operands(M, N, K, "n(0,0.1)", M + 3 * N + 7 * K)
    ref = row_major_result(A, B)
    assert_within_tolerance(ref, oracle.gemm(A, B), f"{M}x{N}x{K} row-major")
    for a_col, b_col, c_col in LAYOUTS:
        Av = place(A, a_col, pad=5)
        Bv = place(B, b_col, pad=3)
        Cv = output(M, N, c_col)
        got = call(Av, Bv, Cv)
        assert np.array_equal(got, ref), (a_col, b_col, c_col)
        assert padding_untouched(Cv, c_col), (a_col, b_col, c_col)


@pytest.mark.parametrize("a_col,b_col", [(False, True), (True, False), (True, True)])
@pytest.mark.parametrize("offsets", [(1, 0), (0, 3), (1, 1), (2, 6)])
def test_transposed_unaligned_and_odd_ld(a_col, b_col, offsets):
    """2-byte-aligned starts and odd leading dimensions, ragged K (head panel) and a 1-column
    sliver, on the DMA path and on the generic path."""
    M, N, K = 700, 513, 333
    A, B = operands(M, N, K, "u(-0.5,0.5)", 17)
    ref = row_major_result(A, B)
    Av = place(A, a_col, pad=1, offset=offsets[0])
    Bv = place(B, b_col, pad=1, offset=offsets[1])
    got = call(Av, Bv, output(M, N, False))
    assert np.array_equal(got, ref)
    gen = call(Av, Bv, output(M, N, False), force_generic=1)
    assert_within_tolerance(gen, oracle.gemm(A, B), f"generic {a_col} {b_col} {offsets}")


@pytest.mark.parametrize("a_col,b_col", [(False, True), (True, False), (True, True)])
def test_last_elements_in_every_order(a_col, b_col):
    """One-hot operands whose only non-zero is the matrix's last stored element, at every
    alignment of the matrix's end: that element is the one the DMA path re-reads."""
    M, N, K = 300, 270, 130
    one = np.float16(1.0).view(np.uint16)
    _, R = operands(M, N, K, "u(-0.5,0.5)", 23)
    for off in range(4):
        # A's last element A[M-1][K-1] = 1 (column-major: that is also its last stored one)
        A = np.zeros((M, K), np.uint16)
        A[M - 1, K - 1] = one
        got = call(place(A, a_col, pad=off, offset=off), place(R, b_col, pad=1, offset=3 - off),
                   output(M, N, False))
        want = np.zeros((M, N), np.uint16)
        want[M - 1] = R[K - 1]
        assert np.array_equal(got, want), ("A", off)
        # B's last element B[K-1][N-1] = 1
        Bz = np.zeros((K, N), np.uint16)
        Bz[K - 1, N - 1] = one
        Ar = operands(M, 1, K, "u(-0.5,0.5)", 29)[0]
        got = call(place(Ar, a_col, pad=1, offset=3 - off), place(Bz, b_col, pad=off, offset=off),
                   output(M, N, False))
        want = np.zeros((M, N), np.uint16)
        want[:, N - 1] = Ar[:, K - 1]
        assert np.array_equal(got, want), ("B", off)


@pytest.mark.parametrize("tile", sorted(g.TILES))
@pytest.mark.parametrize("a_col,b_col", [(False, True), (True, False), (True, True)])
def test_every_tile_in_every_order(tile, a_col, b_col):
    for M, N, K in [(257, 129, 65), (33, 8, 64), (7, 300, 190)]:
        A, B = operands(M, N, K, "n(0,0.1)", 5 * M + N + K)
        ref = row_major_result(A, B, tile=tile)
        got = call(place(A, a_col, pad=2), place(B, b_col, pad=2), output(M, N, False), tile=tile)
        assert np.array_equal(got, ref), (M, N, K)


@pytest.mark.parametrize("a_col,b_col,c_col", [(False, True, False), (True, False, False),
                                               (True, True, False), (False, False, True)])
def test_large_layouts_equal_row_major(a_col, b_col, c_col):
    M = N = K = 4096
    A, B = operands(M, N, K, "u(-0.5,0.5)", 2)
    ref = row_major_result(A, B)
    got = call(place(A, a_col), place(B, b_col), output(M, N, c_col, pad=0))
    assert np.array_equal(got, ref)


def test_matmul_reads_transposed_views():
    """The torch-level call passes strides: w.t() and a column-major output work in place."""
    M, N, K = 384, 320, 256
    A, B = operands(M, N, K, "u(-0.5,0.5)", 31)
    ref = row_major_result(A, B)
    Bt = to_dev(np.ascontiguousarray(B.T))          # N x K, as a linear layer stores weights
    got = from_dev(g.matmul(to_dev(A), Bt.t()))
    assert np.array_equal(got, ref)
    out = torch.empty((N, M), dtype=torch.int16, device="cuda").t()
    g.matmul(to_dev(A), to_dev(B), out)
    assert np.array_equal(from_dev(out), ref)
    with pytest.raises(g.GemmError):
        g.matmul(to_dev(A), to_dev(B)[:, ::2], M=M, N=N // 2, K=K)   # no unit stride


@pytest.mark.parametrize("M,N", [(4095, 1), (4095, 7), (2000, 31), (1, 3000), (9, 2500), (33, 700)])
def test_thin_strips_in_every_order(M, N):
    """Problems narrower than one tile (the shape of split-off edge strips) in every storage
    order: equal to the row-major result bit for bit, and to the oracle within tolerance."""
    K = 1021
    A, B = operands(M, N, K, "n(0,0.1)", M * 3 + N)
    ref = row_major_result(A, B)
    assert_within_tolerance(ref, oracle.gemm(A, B), f"{M}x{N}x{K}")
    for a_col, b_col in [(False, False), (True, False), (False, True), (True, True)]:
        got = call(place(A, a_col, pad=3), place(B, b_col, pad=3), output(M, N, False))
        assert np.array_equal(got, ref), (a_col, b_col)


# Unpadded operands (ld equal to the stored row length) with NaN or Inf right after their last
# element.  A buffer resource's extent is rounded up to a whole dword, so for an x-major operand
# (B row-major, A column-major) with an odd number of elements from the last panel's corner it
# admits that next element, at row k = K, x = 0; a path that stages rows k >= K must not let it
# in, since Inf or NaN times the zero it meets there is NaN (row or column 0 of C would be NaN).
# K is odd in every shape, and so is the x extent of at least one operand; (2, 1, 1301) is
# planned with B as a 1-wide row-major operand.
TIGHT_SHAPES = [(87, 317, 679), (2, 1, 1301), (649, 687, 215), (30, 341, 1), (563, 217, 1011),
                (5, 7, 3)]


@pytest.mark.parametrize("fill", [0x7E00, 0x7C00], ids=["nan", "inf"])
@pytest.mark.parametrize("M,N,K", TIGHT_SHAPES)
def test_unpadded_operands_ignore_what_follows_them(M, N, K, fill):
    A, B = operands(M, N, K, "n(0,0.1)", 11 * M + N + K)
    want = oracle.gemm(A, B)
    for a_col, b_col, c_col in LAYOUTS:
        Av = place(A, a_col, pad=0, fill=fill)
        Bv = place(B, b_col, pad=0, fill=fill)
        for generic in (0, 1):
            what = f"{M}x{N}x{K} cols={a_col, b_col, c_col} generic={generic}"
            Cv = output(M, N, c_col)
            got = call(Av, Bv, Cv, force_generic=generic)
            assert_within_tolerance(got, want, what)
            assert padding_untouched(Cv, c_col), what


@pytest.mark.parametrize("tile", sorted(g.TILES))
def test_identity_through_every_tile_and_order(tile):
    # A I = A and I B = B exactly, for every storage order of A and B, on the DMA and the
    # generic path: every element must travel through the LDS layouts (swizzles, transposing
    # reads), the MFMA lane map and the store to its own place.  Sizes are ragged against
    # every tile (200 rows, 136 = 2 x 64 + 8 k values, 72 columns).
    M, K, N = 200, 136, 72
    A, _ = operands(M, 1, K, "n(0,0.1)", 31)
    _, B = operands(1, N, K, "n(0,0.1)", 37)
    eye = np.eye(K, dtype=np.float16).view(np.uint16)
    for a_col, b_col in itertools.product((False, True), repeat=2):
        for generic in (0, 1):
            what = f"tile {tile} cols={a_col, b_col} generic={generic}"
            got = call(place(A, a_col, pad=1), place(eye, b_col, pad=3), output(M, K, False),
                       tile=tile, force_generic=generic)
            assert np.array_equal(got, A), "A I " + what
            got = call(place(eye, a_col, pad=2), place(B, b_col), output(K, N, True),
                       tile=tile, force_generic=generic)
            assert np.array_equal(got, B), "I B " + what
