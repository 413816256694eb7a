"""Randomized GPU parity: seeded random problems across the whole option space.

Each case draws from a fixed-seed generator: M, N in 1..700 and K in 0..3000 (half of the
draws log-uniform, half uniform from 64), each matrix's storage order (row- or column-major),
its leading-dimension padding (0..5 elements) and start offset (0..3 elements, so 2-byte
aligned starts occur), the operand distribution, and the options -- tile (automatic or any of the 16), GROUP_SIZE_M, XCD
remap, persistent schedule, edge split, the generic path, split K (none, 2..9 slices, or the
automatic choice).  Every result must meet the 1e-2 + 2^-10 |oracle| bar against the oracle
(matmul of phobos "03: Matrix multiplication": fp32 accumulation, one fp16 narrowing), C's
padding must keep its canary, and where neither the generic path nor split K is used the
result must be the default row-major call's, bit for bit (tiles, group sizes, the remap, the
schedule, the edge split and storage orders never change a bit).
"""
import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import (assert_within_tolerance, from_dev, output, padding_untouched, place,
                      to_dev)
from synthetic_inputs import DISTS, operands

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

CASES = 1000


def log_uniform(rng, lo, hi):
    return int(round(np.exp(rng.uniform(np.log(lo), np.log(hi)))))


def draw_case(case):
    rng = np.random.default_rng(1000 + case)

    def size(hi):   # half the draws log-uniform from 1 (edge shapes), half uniform from 64
        return log_uniform(rng, 1, hi) if rng.random() < 0.5 else int(rng.integers(64, hi + 1))
    M, N = size(700), size(700)
    K = 0 if rng.random() < 0.03 else size(3000)
    layout = [bool(rng.integers(2)) for _ in range(3)]          # A, B, C column-major
    pads = [int(rng.integers(0, 6)) for _ in range(3)]
    offs = [int(rng.integers(0, 4)) for _ in range(2)]
    dist = DISTS[int(rng.integers(len(DISTS)))]
    opts = {}
    if rng.random() < 0.5:
        opts["tile"] = int(rng.choice(sorted(g.TILES)))
    if rng.random() < 0.3:
        opts["group_m"] = int(rng.integers(1, 17))
    if rng.random() < 0.3:
        opts["xcd_remap"] = int(rng.integers(0, 3))
    if rng.random() < 0.3:
        opts["split_edges"] = int(rng.integers(0, 3))
    r = rng.random()
    if r < 0.25:
        opts["split_k"] = int(rng.integers(2, 10))
    elif r < 0.35:
        opts["split_k"] = g.SPLIT_K_AUTO
    elif r < 0.45:
        opts["force_generic"] = 1
    if "split_k" not in opts and rng.random() < 0.25:
        opts["persistent"] = g.PERSISTENT_ON
    return M, N, K, layout, pads, offs, dist, opts


@pytest.mark.parametrize("case", range(CASES))
def test_random_case(case):
    M, N, K, (a_col, b_col, c_col), (pa, pb, pc), (oa, ob), dist, opts = draw_case(case)
    what = f"case {case}: {M}x{N}x{K} {dist} cols={a_col, b_col, c_col} opts={opts}"
    print(what, flush=True)
    A, B = operands(M, N, K, dist, case)
    Av = place(A, a_col, pad=pa, offset=oa)
    Bv = place(B, b_col, pad=pb, offset=ob)
    Cv = output(M, N, c_col, pad=pc)
    g.matmul(Av, Bv, Cv, **opts)
    got = from_dev(Cv)
    assert padding_untouched(Cv, c_col), what
    assert_within_tolerance(got, oracle.gemm(A, B), what)
    if "split_k" not in opts and "force_generic" not in opts:
        ref = from_dev(g.matmul(to_dev(A), to_dev(B)))
        assert np.array_equal(got, ref), what
