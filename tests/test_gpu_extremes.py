"""GPU parity at the extremes of the shape space: very deep K and very long, thin C.

* K = 2^17 (2048 panels of 64, a 131072-deep fp32 sum per element; K + 5 for a head panel)
  with M = N = 64, unsplit and split K: every element against the oracle.
* M or N = 10^6 with the other side 2..33 and short K: grids of tens of thousands of
  workgroups on a 1-D launch, the last tile row / column ragged, both storage orders of C.
* A leading dimension of 2^24 + 8 elements (a 33.6 GB operand buffer), where the choice of
  tile depends on the kernels' 32-bit offsets.
The bar is the usual 1e-2 + 2^-10 |oracle| (matmul of phobos "03: Matrix multiplication":
fp32 accumulation, one fp16 narrowing); unsplit results must not depend on the tile.
"""
import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import assert_within_tolerance, from_dev, to_dev
from synthetic_inputs import operands

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("K", [1 << 17, (1 << 17) + 5])
def test_very_deep_k(K):
    M = N = 64
    A, B = operands(M, N, K, "u(-0.5,0.5)", 17)
    want = oracle.gemm(A, B)
    Ad, Bd = to_dev(A), to_dev(B)
    plain = from_dev(g.matmul(Ad, Bd))
    assert_within_tolerance(plain, want, f"64x64x{K}")
    assert np.array_equal(plain, from_dev(g.matmul(Ad, Bd, tile=g.TILE_32x32x128)))
    for S in (16, g.SPLIT_K_AUTO):
        split = from_dev(g.matmul(Ad, Bd, split_k=S))
        assert_within_tolerance(split, want, f"64x64x{K} split {S}")


@pytest.mark.parametrize("M,N,K", [(1_000_000, 2, 16), (3, 1_000_000, 40), (999_999, 33, 8)])
def test_very_long_thin_c(M, N, K):
    A, B = operands(M, N, K, "n(0,0.1)", M % 1000 + N)
    want = oracle.gemm(A, B)
    Ad, Bd = to_dev(A), to_dev(B)
    got = from_dev(g.matmul(Ad, Bd))
    assert_within_tolerance(got, want, f"{M}x{N}x{K}")
    rc, info = g.gemm_f16f32_plan(M, N, K, Ad.data_ptr(), Bd.data_ptr(), 1 << 40, K, N, N)
    assert rc == g.OK and info["num_programs"] >= 1000
    # column-major C (computed as C^T = B^T A^T) gives the same bits
    Ct = torch.empty((N, M), dtype=torch.int16, device="cuda")
    g.matmul(Ad, Bd, Ct.t())
    assert np.array_equal(from_dev(Ct).T, got)


def test_leading_dimension_past_a_deep_panels_offsets():
    # B row-major with ldb = 2^24 + 8 (a 33.6 GB buffer, NaN outside B's 32 columns): one
    # 128-deep panel spans 128 ldb > 2^31 elements, past the kernels' 32-bit offsets, while a
    # 64-deep one does not.  The planner's own choice for 32 x 32 x 1000 is a 128-deep tile; it
    # gives way to the 32 x 32 x 64 tile, and a forced 128-deep tile is refused.
    M, N, K = 32, 32, 1000
    ld = (1 << 24) + 8
    A, B = operands(M, N, K, "n(0,0.1)", 23)
    buf = torch.full((K * ld,), 0x7E00, dtype=torch.int16, device="cuda")
    try:
        Bv = buf.view(K, ld)[:, :N]
        Bv.copy_(to_dev(B))
        Ad = to_dev(A)
        rc, info = g.gemm_f16f32_plan(M, N, K, Ad.data_ptr(), Bv.data_ptr(), 1 << 40, K, ld, N)
        assert rc == g.OK and info["tile"] == g.TILE_32x32x64
        assert_within_tolerance(from_dev(g.matmul(Ad, Bv)), oracle.gemm(A, B), "ldb 2^24+8")
        with pytest.raises(g.GemmError):
            g.matmul(Ad, Bv, tile=g.TILE_32x64x128)
    finally:
        del buf
        torch.cuda.empty_cache()
