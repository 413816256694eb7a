"""GPU parity of split K (opts.split_k through gemm_f16f32_strided_ws).

Split K cuts the k range into slices of L = roundup(cdiv(K, S), 128) values from the end of
k; each slice's fp32 tile sums go to the workspace and a second kernel adds the slices in
order and narrows once, so C is still the fp32 sum of A[i][k] B[k][j] rounded once to fp16
(matmul of phobos "03: Matrix multiplication": fp32 accumulator, one `.to(float16)` at the
end), only summed in another order.  Checks: every result within 1e-2 + 2^-10 |oracle| of
the oracle; exact integer sums equal to the oracle bit for bit; one result for every tile
and every storage order at a given S (the slices do not depend on the tile); run-to-run
determinism; nothing written outside C's M x N block and the planned workspace bytes.
"""
import itertools

import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import (assert_within_tolerance, checksum_ok, from_dev, output, padding_untouched,
                      place, sample_positions, to_dev)
from synthetic_inputs import operands

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WS_CANARY = 0x5A


def args_of(Av, Bv, Cv):
    M, K = Av.shape
    N = Bv.shape[1]
    return (M, N, K, Av.data_ptr(), Av.stride(0), Av.stride(1), Bv.data_ptr(), Bv.stride(0),
            Bv.stride(1), Cv.data_ptr(), Cv.stride(0), Cv.stride(1))


def split_plan(Av, Bv, Cv, **opts):
    rc, info = g.gemm_f16f32_strided_plan(*args_of(Av, Bv, Cv), opts=opts)
    assert rc == g.OK, g.gemm_f16f32_strerror(rc)
    return info


def split_call(Av, Bv, Cv, ws=None, **opts):
    """C through gemm_f16f32_strided_ws; ws: a uint8 CUDA tensor (default: exactly the
    planned size).  Returns (C bits, plan)."""
    info = split_plan(Av, Bv, Cv, **opts)
    if ws is None:
        ws = torch.empty(max(info["workspace_bytes"], 16), dtype=torch.uint8, device="cuda")
    rc = g.gemm_f16f32_strided_ws(*args_of(Av, Bv, Cv), ws.data_ptr(), ws.numel(),
                                  torch.cuda.current_stream().cuda_stream, opts)
    assert rc == g.OK, g.gemm_f16f32_strerror(rc)
    return from_dev(Cv), info


def row_major(A, B):
    return place(A, False), place(B, False)


@pytest.mark.parametrize("M,N,K,S,dist", [
    (64, 64, 4096, 2, "u(-0.5,0.5)"), (64, 64, 4096, 4, "n(0,0.1)"),
    (64, 64, 4096, 32, "u(-0.5,0.5)"), (300, 264, 2000, 3, "u(0,1)"),
    (129, 65, 4093, 5, "n(0,0.1)"), (1, 1, 1000, 4, "u(-0.5,0.5)"),
    (33, 17, 640, 5, "u(0,1)"), (256, 256, 8192, 16, "u(-0.5,0.5)"),
    (1000, 600, 1500, 4, "n(0,0.1)"), (2, 3, 129, 2, "u(-0.5,0.5)")])
def test_split_within_tolerance(M, N, K, S, dist):
    A, B = operands(M, N, K, dist, M + 7 * N + K + S)
    Av, Bv = row_major(A, B)
    C, info = split_call(Av, Bv, output(M, N, False), split_k=S)
    assert info["splits"] >= 2
    assert_within_tolerance(C, oracle.gemm(A, B), f"{M}x{N}x{K} split {S}")


@pytest.mark.parametrize("S", [2, 3, 8, 31])
def test_split_exact_integer_sums(S):
    """Integers in [-2, 2]: every partial sum is an integer below 2^24, exact in fp32 in any
    order, so the split result is the oracle's single rounding bit for bit (sums beyond 2048
    also exercise the fp16 rounding of large integers)."""
    M, N, K = 96, 80, 4000
    rng = np.random.default_rng(S)
    A = rng.integers(-2, 3, (M, K)).astype(np.float16).view(np.uint16)
    B = rng.integers(-2, 3, (K, N)).astype(np.float16).view(np.uint16)
    B[:, 0] = np.float16(2.0).view(np.uint16)     # column 0: sums up to +-16000
    A[0, :] = np.float16(2.0).view(np.uint16)
    Av, Bv = row_major(A, B)
    C, _ = split_call(Av, Bv, output(M, N, False), split_k=S)
    assert np.array_equal(C, oracle.gemm(A, B))


def test_every_tile_gives_the_same_split_result():
    M, N, K, S = 200, 150, 1500, 3
    A, B = operands(M, N, K, "n(0,0.1)", 5)
    Av, Bv = row_major(A, B)
    ref = None
    for t in sorted(g.TILES):
        C, info = split_call(Av, Bv, output(M, N, False), split_k=S, tile=t)
        assert info["tile"] == t and info["splits"] == 3
        if ref is None:
            ref = C
            assert_within_tolerance(C, oracle.gemm(A, B), "split 3")
        assert np.array_equal(C, ref), t


@pytest.mark.parametrize("a_col,b_col,c_col", list(itertools.product((False, True), repeat=3)))
def test_every_storage_order_gives_the_same_split_result(a_col, b_col, c_col):
    """Row- or column-major operands and C, odd leading dimensions and 2-byte aligned starts:
    one result, bit for bit (a column-major C is computed as C^T = B^T A^T)."""
    M, N, K, S = 301, 203, 1100, 3
    A, B = operands(M, N, K, "u(-0.5,0.5)", 9)
    ref, _ = split_call(*row_major(A, B), output(M, N, False), split_k=S)
    assert_within_tolerance(ref, oracle.gemm(A, B), "split row-major")
    for pad, off in ((0, 0), (1, 1)):
        Av = place(A, a_col, pad=pad, offset=off)
        Bv = place(B, b_col, pad=pad, offset=off)
        Cv = output(M, N, c_col)
        got, info = split_call(Av, Bv, Cv, split_k=S)
        assert info["swapped"] == int(c_col)
        assert np.array_equal(got, ref), (pad, off)
        assert padding_untouched(Cv, c_col)


def test_workspace_bounds_reuse_and_determinism():
    """Nothing past the planned workspace bytes is written; a workspace reused for another
    (smaller) problem gives that problem's result; repeated calls agree bit for bit."""
    M, N, K, S = 130, 70, 3000, 6
    A, B = operands(M, N, K, "n(0,0.1)", 13)
    Av, Bv = row_major(A, B)
    need = split_plan(Av, Bv, output(M, N, False), split_k=S)["workspace_bytes"]
    ws = torch.full((need + 4096,), WS_CANARY, dtype=torch.uint8, device="cuda")
    C1, _ = split_call(Av, Bv, output(M, N, False), ws=ws, split_k=S)
    C2, _ = split_call(Av, Bv, output(M, N, False), ws=ws, split_k=S)
    assert np.array_equal(C1, C2)
    assert bool((ws[need:] == WS_CANARY).all())
    assert_within_tolerance(C1, oracle.gemm(A, B), "split 6")
    # a smaller problem in the same workspace
    m, n, k = 40, 33, 700
    a, b = operands(m, n, k, "u(-0.5,0.5)", 14)
    c, info = split_call(*row_major(a, b), output(m, n, False), ws=ws, split_k=3)
    assert info["splits"] == 3 and info["workspace_bytes"] < need
    assert_within_tolerance(c, oracle.gemm(a, b), "split 3 after split 6")


def test_no_split_leaves_the_workspace_alone():
    """K within one slice: no split; the call is the plain one, bit for bit."""
    M, N, K = 100, 90, 128
    A, B = operands(M, N, K, "u(-0.5,0.5)", 15)
    Av, Bv = row_major(A, B)
    ws = torch.full((1 << 16,), WS_CANARY, dtype=torch.uint8, device="cuda")
    C, info = split_call(Av, Bv, output(M, N, False), ws=ws, split_k=4)
    assert info["splits"] == 1
    assert bool((ws == WS_CANARY).all())
    assert np.array_equal(C, from_dev(g.matmul(to_dev(A), to_dev(B))))


def test_matmul_allocates_the_workspace():
    M, N, K = 128, 96, 2048
    A, B = operands(M, N, K, "u(-0.5,0.5)", 16)
    C = from_dev(g.matmul(to_dev(A), to_dev(B), split_k=4))
    ref, _ = split_call(*row_major(A, B), output(M, N, False), split_k=4)
    assert np.array_equal(C, ref)


def test_large_split_sampled():
    """2048 x 2048 x 8192 in 4 slices: sampled elements against the oracle, and checksums."""
    M, N, K, S = 2048, 2048, 8192, 4
    A, B = operands(M, N, K, "u(-0.5,0.5)", 3)
    Av, Bv = row_major(A, B)
    C, info = split_call(Av, Bv, output(M, N, False, pad=0), split_k=S)
    assert info["splits"] == S
    r, c = sample_positions(M, N, info["bm"], info["bn"], 4, 7)
    assert_within_tolerance(C[r, c], oracle.gemm_sampled(A, B, r, c), "2048^2 x 8192 split 4")
    assert checksum_ok(A, B, C)


def test_graph_capture_replays_match_eager():
    """The two launches of a split call captured in a HIP graph (neither uses a memset):
    every replay, with eager work between replays, reproduces the eager result."""
    M, N, K, S = 256, 192, 4096, 4
    A, B = operands(M, N, K, "n(0,0.1)", 17)
    Ad, Bd = to_dev(A), to_dev(B)
    C = torch.empty((M, N), dtype=torch.int16, device="cuda")
    ws = torch.empty(S * M * N * 4, dtype=torch.uint8, device="cuda")
    eager = from_dev(g.matmul(Ad, Bd, C, workspace=ws, split_k=S))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(graph, stream=s):
            g.matmul(Ad, Bd, C, workspace=ws, split_k=S)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        C.fill_(0)
        ws.fill_(WS_CANARY)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(C), eager), rep


def test_automatic_split_matches_its_explicit_choice():
    """split_k = SPLIT_K_AUTO with a workspace runs the planned split, bit for bit the explicit
    call with that S; without room in the workspace, or through the entry points that take
    none, the call runs unsplit (and never touches the workspace)."""
    M, N, K = 64, 64, 8192
    A, B = operands(M, N, K, "u(-0.5,0.5)", 21)
    Av, Bv = row_major(A, B)
    auto = split_plan(Av, Bv, output(M, N, False), split_k=g.SPLIT_K_AUTO)
    S = auto["splits"]
    assert S >= 4
    explicit, _ = split_call(Av, Bv, output(M, N, False), split_k=S)
    got, _ = split_call(Av, Bv, output(M, N, False), split_k=g.SPLIT_K_AUTO)
    assert np.array_equal(got, explicit)
    assert_within_tolerance(got, oracle.gemm(A, B), "automatic split")
    via_matmul = from_dev(g.matmul(to_dev(A), to_dev(B), workspace=torch.empty(
        auto["workspace_bytes"], dtype=torch.uint8, device="cuda")))
    assert np.array_equal(via_matmul, explicit)
    unsplit = from_dev(g.matmul(to_dev(A), to_dev(B)))
    small = torch.full((auto["workspace_bytes"] - 16,), WS_CANARY, dtype=torch.uint8,
                       device="cuda")
    got_small, _ = split_call(Av, Bv, output(M, N, False), ws=small, split_k=g.SPLIT_K_AUTO)
    assert np.array_equal(got_small, unsplit)
    assert bool((small == WS_CANARY).all())
    Cv = output(M, N, False)
    rc = g.gemm_f16f32_strided(*args_of(Av, Bv, Cv), torch.cuda.current_stream().cuda_stream,
                               dict(split_k=g.SPLIT_K_AUTO))
    assert rc == g.OK
    assert np.array_equal(from_dev(Cv), unsplit)


def test_matmul_on_a_side_stream_keeps_its_workspace():
    """matmul(stream=side) with split K and no workspace: the workspace (and `out`) are
    allocated on the side stream, so memory the current stream allocates and writes right
    after the call -- while the side stream's kernels may still run -- is never the
    workspace.  The result must equal the same call on the current stream."""
    M, N, K = 128, 128, 8192
    A, B = operands(M, N, K, "u(-0.5,0.5)", 77)
    Ad, Bd = to_dev(A), to_dev(B)
    want = from_dev(g.matmul(Ad, Bd, split_k=8))
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for rep in range(3):
        C = g.matmul(Ad, Bd, split_k=8, stream=side)
        junk = [torch.full((1 << 20,), 0x7E00 + rep, dtype=torch.int16, device="cuda")
                for _ in range(8)]
        torch.cuda.current_stream().wait_stream(side)
        got = from_dev(C)
        assert np.array_equal(got, want), rep
        del junk
    assert_within_tolerance(want, oracle.gemm(A, B), "split K on a side stream")
