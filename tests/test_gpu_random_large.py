"""Randomized GPU parity on large problems: seeded draws with M, N up to 5000 and K up to 6000
(60 % of the draws uniform from 256, the rest log-uniform from 1), every storage order, leading-
dimension padding of 0, 1, 3 or 64 elements, 2-byte aligned starts, NaN or Inf in the operands'
padding and after their last element, and the whole option space (tile, GROUP_SIZE_M, XCD remap,
edge split, persistent schedule, generic path, split K).  The oracle is sampled: the four
corners of every 256 x 256 block of C and four random elements in each (matmul of phobos "03:
Matrix multiplication": fp32 accumulation, one fp16 narrowing; bar 1e-2 + 2^-10 |oracle|).
Where neither the generic path nor split K runs, the whole result must equal the default
row-major call bit for bit, and C's padding must keep its canary in every case.
"""
import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import (assert_within_tolerance, from_dev, output, padding_untouched, place,
                      sample_positions, to_dev)
from synthetic_inputs import DISTS, operands

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = 60


def draw_case(case):
    rng = np.random.default_rng(50000 + case)
    big = rng.random() < 0.6

    def size(hi):
        if big:
            return int(rng.integers(256, hi + 1))
        return int(round(np.exp(rng.uniform(0.0, np.log(hi)))))
    M, N = size(5000), size(5000)
    K = 0 if rng.random() < 0.02 else size(6000)
    layout = [bool(rng.integers(2)) for _ in range(3)]      # A, B, C column-major
    pads = [int(rng.choice([0, 0, 1, 3, 64])) for _ in range(3)]
    offs = [int(rng.integers(0, 4)) for _ in range(2)]
    dist = DISTS[int(rng.integers(len(DISTS)))]
    fill = int(rng.choice([0x7E00, 0x7C00]))                 # NaN or +Inf around A and B
    opts = {}
    if rng.random() < 0.4:
        opts["tile"] = int(rng.choice(sorted(g.TILES)))
    if rng.random() < 0.3:
        opts["group_m"] = int(rng.integers(1, 33))
    if rng.random() < 0.3:
        opts["xcd_remap"] = int(rng.integers(0, 3))
    if rng.random() < 0.3:
        opts["split_edges"] = int(rng.integers(0, 3))
    r = rng.random()
    if r < 0.2:
        opts["split_k"] = int(rng.integers(2, 17))
    elif r < 0.35:
        opts["split_k"] = g.SPLIT_K_AUTO
    elif r < 0.45:
        opts["force_generic"] = 1
    if "split_k" not in opts and rng.random() < 0.25:
        opts["persistent"] = g.PERSISTENT_ON
    return M, N, K, layout, pads, offs, dist, fill, opts


@pytest.mark.parametrize("case", range(CASES))
def test_random_large_case(case):
    M, N, K, (a_col, b_col, c_col), (pa, pb, pc), (oa, ob), dist, fill, opts = draw_case(case)
    what = (f"case {case}: {M}x{N}x{K} {dist} cols={a_col, b_col, c_col} pads={pa, pb, pc} "
            f"offs={oa, ob} fill={fill:#06x} opts={opts}")
    print(what, flush=True)
    A, B = operands(M, N, K, dist, case)
    Av = place(A, a_col, pad=pa, offset=oa, fill=fill)
    Bv = place(B, b_col, pad=pb, offset=ob, fill=fill)
    Cv = output(M, N, c_col, pad=pc)
    g.matmul(Av, Bv, Cv, **opts)
    got = from_dev(Cv)
    assert padding_untouched(Cv, c_col), what
    rows, cols = sample_positions(M, N, 256, 256, 4, case)
    assert_within_tolerance(got[rows, cols], oracle.gemm_sampled(A, B, rows, cols), what)
    if "split_k" not in opts and "force_generic" not in opts:
        ref = from_dev(g.matmul(to_dev(A), to_dev(B)))
        assert np.array_equal(got, ref), what
