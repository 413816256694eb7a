"""gemm_f16f32_strided_scratch: split K for callers that cannot allocate device memory.

The entry point keeps its fp32 slices in the library's static device array instead of a
caller workspace; it must give, bit for bit, what gemm_f16f32_strided_ws gives with a
workspace of its own (same plan, same kernels, slices added in the same order), and both
must meet the oracle's bar.  Two calls in a row, the second smaller, check that what the
first left in the array does not leak into the second.
"""
import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import assert_within_tolerance, from_dev, to_dev
from synthetic_inputs import operands

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def strided_args(Ad, Bd, Cd, M, N, K):
    return (M, N, K, Ad.data_ptr(), Ad.stride(0), Ad.stride(1), Bd.data_ptr(), Bd.stride(0),
            Bd.stride(1), Cd.data_ptr(), Cd.stride(0), Cd.stride(1))


def both_entry_points(M, N, K, seed, split_k):
    A, B = operands(M, N, K, "u(-0.5,0.5)", seed)
    Ad, Bd = to_dev(A), to_dev(B)
    stream = torch.cuda.current_stream().cuda_stream
    opts = dict(split_k=split_k)
    C_ws = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda")
    rc, info = g.gemm_f16f32_strided_plan(*strided_args(Ad, Bd, C_ws, M, N, K), opts=opts)
    assert rc == g.OK and info["splits"] > 1, info
    assert 0 < info["workspace_bytes"] <= g.SCRATCH_BYTES
    ws = torch.empty(info["workspace_bytes"], dtype=torch.uint8, device="cuda")
    rc = g.gemm_f16f32_strided_ws(*strided_args(Ad, Bd, C_ws, M, N, K), ws.data_ptr(),
                                  ws.numel(), stream, opts)
    assert rc == g.OK, g.gemm_f16f32_strerror(rc)
    C_sc = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda")
    rc = g.gemm_f16f32_strided_scratch(*strided_args(Ad, Bd, C_sc, M, N, K), stream, opts)
    assert rc == g.OK, g.gemm_f16f32_strerror(rc)
    torch.cuda.synchronize()
    return A, B, from_dev(C_ws), from_dev(C_sc), info


def test_scratch_matches_workspace_entry_two_calls():
    """Call 1: 256 x 512 x 8192 in 8 slices (4 MiB of scratch); call 2, right after:
    96 x 160 x 3000 in 4 slices (a smaller, ragged problem over the first call's leftovers)."""
    for (M, N, K, seed, S) in [(256, 512, 8192, 41, 8), (96, 160, 3000, 42, 4)]:
        print(f"scratch split K: {M}x{N}x{K}, split_k {S}", flush=True)
        A, B, C_ws, C_sc, info = both_entry_points(M, N, K, seed, S)
        assert np.array_equal(C_sc, C_ws), (M, N, K)
        assert_within_tolerance(C_sc, oracle.gemm(A, B), f"{M}x{N}x{K} scratch")


def test_scratch_automatic_split_and_unsplit_calls():
    """SPLIT_K_AUTO through the scratch entry point equals the workspace entry point; a shape
    that is not split runs as gemm_f16f32_strided."""
    M, N, K = 64, 64, 8192
    A, B, C_ws, C_sc, info = both_entry_points(M, N, K, 43, g.SPLIT_K_AUTO)
    assert np.array_equal(C_sc, C_ws)
    assert_within_tolerance(C_sc, oracle.gemm(A, B), "auto split scratch")
    M, N, K = 300, 264, 200
    A, B = operands(M, N, K, "u(-0.5,0.5)", 44)
    Ad, Bd = to_dev(A), to_dev(B)
    C = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    rc = g.gemm_f16f32_strided_scratch(*strided_args(Ad, Bd, C, M, N, K),
                                       torch.cuda.current_stream().cuda_stream, None)
    assert rc == g.OK
    assert np.array_equal(from_dev(C), from_dev(g.matmul(Ad, Bd)))


def test_scratch_refuses_a_split_larger_than_the_array():
    """16 slices of 1024 x 1024 need 64 MiB of fp32 partials: refused before any launch, C
    untouched."""
    M = N = 1024
    K = 8192
    Ad = torch.zeros((M, K), dtype=torch.int16, device="cuda")
    Bd = torch.zeros((K, N), dtype=torch.int16, device="cuda")
    C = torch.full((M, N), 0x1234, dtype=torch.int16, device="cuda")
    rc, info = g.gemm_f16f32_strided_plan(*strided_args(Ad, Bd, C, M, N, K),
                                          opts=dict(split_k=16))
    assert rc == g.OK and info["workspace_bytes"] > g.SCRATCH_BYTES
    rc = g.gemm_f16f32_strided_scratch(*strided_args(Ad, Bd, C, M, N, K),
                                       torch.cuda.current_stream().cuda_stream,
                                       dict(split_k=16))
    assert rc == g.ERR_SCRATCH
    torch.cuda.synchronize()
    assert bool((C == 0x1234).all())
