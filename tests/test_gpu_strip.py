"""GPU parity of the ping-pong tile's strip: a last tile column of 1-16 columns computed inside
the main launch (plan_info.strip_n), by the tile rows' own workgroups.

Every case is compared with the oracle at every element (matmul of phobos "03: Matrix
multiplication": fp32 accumulation, one fp16 narrowing; tolerance 1e-2 + 2^-10 |oracle|) and,
bit for bit, with the same call with the edge split off, where the strip's columns are
ordinary columns of a 17th tile column: both add each element's products in the same
sequence of 32-deep MFMA steps.  Covered: strip widths 1-16, B stored row-major (the strip
staged as k rows) and column-major (as strip rows of k), K with and without a head panel,
K within one panel, odd leading dimensions, and C's padding left untouched.
"""
import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import assert_within_tolerance, from_dev, output, padding_untouched, place
from synthetic_inputs import operands

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

PP = dict(tile=g.TILE_256x256x32_PP, split_edges=g.SPLIT_ON)


@pytest.mark.parametrize("M,w,K,b_col,pads", [
    (300, 1, 4093, False, (1, 1)),
    (300, 1, 4093, True, (1, 1)),
    (257, 7, 1000, False, (0, 3)),
    (512, 8, 37, False, (1, 0)),
    (300, 9, 20, True, (3, 1)),
    (300, 16, 96, False, (0, 0)),
    (300, 16, 95, True, (0, 0)),
    (1000, 3, 2, False, (1, 1)),
    (4095, 1, 513, False, (1, 1)),
])
def test_strip_inside_the_main_launch(M, w, K, b_col, pads):
    N = 4096 + w
    what = f"{M}x{N}x{K} B {'column' if b_col else 'row'}-major, pads {pads}"
    print(what, flush=True)
    A, B = operands(M, N, K, "n(0,0.1)", M + w + K)
    Av = place(A, False, pad=pads[0])
    Bv = place(B, b_col, pad=pads[1])
    Cv = output(M, N, False, pad=3)
    rc, info = g.gemm_f16f32_strided_plan(M, N, K, Av.data_ptr(), *Av.stride(), Bv.data_ptr(),
                                          *Bv.stride(), Cv.data_ptr(), *Cv.stride(), opts=PP)
    assert rc == g.OK and info["strip_n"] == w and info["launches"] == 1, info
    g.matmul(Av, Bv, Cv, **PP)
    got = from_dev(Cv)[:M, :N]
    assert padding_untouched(Cv, False), what
    assert_within_tolerance(got, oracle.gemm(A, B), what)
    whole = from_dev(g.matmul(Av, Bv, tile=g.TILE_256x256x32_PP, split_edges=g.SPLIT_OFF))
    assert np.array_equal(got, whole), what


def test_strip_run_to_run_and_default_plan():
    """The ragged workload's shape takes the strip by default (odd leading dimensions); two
    launches give the same bits, equal to the run with the edge split off."""
    M, N, K = 4095, 4097, 4093
    A, B = operands(M, N, K, "n(0,0.1)", 4)
    Ad = place(A, False)
    Bd = place(B, False)
    rc, info = g.gemm_f16f32_strided_plan(M, N, K, Ad.data_ptr(), *Ad.stride(), Bd.data_ptr(),
                                          *Bd.stride(), 3 << 40, N, 1)
    assert rc == g.OK and info["strip_n"] == 1 and info["launches"] == 1
    first = from_dev(g.matmul(Ad, Bd))
    second = from_dev(g.matmul(Ad, Bd))
    assert np.array_equal(first, second)
    assert np.array_equal(first, from_dev(g.matmul(Ad, Bd, split_edges=g.SPLIT_OFF)))
