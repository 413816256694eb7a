"""GPU parity: the HIP path, called through the C-ABI, against the CPU oracle.

Every element of C is compared with the oracle on all five workloads (512^3, 1024x768x128,
4096^3, 8192^3 and 4095x4097x4093) and on many small and ragged shapes; row and column
checksums are an extra check on the large ones.  The tolerance is 1e-2 + 2^-10 |oracle| element-wise; results that have one correct value (the
tile map, closed-form sums exact in fp32, runs that must repeat the same fp32 order) are
compared bit for bit.
"""
import numpy as np
import pytest

import dense_gemm_f16f32_amd as g
import oracle
from gpu_util import assert_within_tolerance, checksum_ok, from_dev, sample_positions, to_dev
from synthetic_inputs import operands, workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def run(A_dev, B_dev, M, N, K, C_dev=None, **opts):
    return g.matmul(A_dev, B_dev, C_dev, M=M, N=N, K=K, **opts)


@pytest.fixture(scope="module", autouse=True)
def _sync_after():
    yield
    torch.cuda.synchronize()


# ---------------------------------------------------------------------------------------
# Tile map: bit-exact against the oracle's grouped map and XCD permutation.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("m,n,G", [(8, 12, 2), (16, 16, 8), (16, 17, 6), (32, 32, 8), (1, 1, 1),
                                   (3, 7, 5), (40, 33, 7), (5, 3, 3), (64, 64, 4),
                                   # large grids and divisors: the map divides by G num_pid_n,
                                   # G and the last group's rows with multiply-and-shift
                                   (1021, 1031, 13), (3, 200001, 2), (700, 3, 1 << 30),
                                   (50000, 41, 7), (46341, 3, 46339)])
@pytest.mark.parametrize("remap", [g.REMAP_ON, g.REMAP_OFF])
def test_tile_map_bit_exact(m, n, G, remap):
    got = g.tile_map(m, n, G, remap).cpu().numpy().astype(np.int64)
    want = oracle.program_tiles(m, n, G, remap == g.REMAP_ON)
    assert np.array_equal(got, want)


def test_huge_group_m_maps_like_one_group():
    """GROUP_SIZE_M beyond the tile rows -- here 2^30, whose product with the 25 tile columns
    would not fit in 32 bits -- maps every program as one group of all the rows does."""
    M, N, K = 600, 800, 96
    A, B = operands(M, N, K, "n(0,0.1)", 17)
    Ad, Bd = to_dev(A), to_dev(B)
    t = g.TILE_32x32x64
    rc, info = g.gemm_f16f32_plan(M, N, K, 1 << 40, 2 << 40, 3 << 40, K, N, N,
                                  opts={"tile": t, "group_m": 1 << 30})
    assert rc == g.OK and info["group_m"] == 1 << 30 and info["num_pid_n"] == 25
    huge = from_dev(run(Ad, Bd, M, N, K, tile=t, group_m=1 << 30))
    whole = from_dev(run(Ad, Bd, M, N, K, tile=t, group_m=info["num_pid_m"]))
    assert np.array_equal(huge, whole)
    assert_within_tolerance(huge, oracle.gemm(A, B), "group_m 2^30")


def test_tile_map_worked_example():
    """1024x768 with 128x64 tiles and G = 2: 96 programs, program 60 -> (4, 6)."""
    t = g.tile_map(8, 12, 2, g.REMAP_OFF).cpu().numpy()
    assert t.shape == (96, 3) and tuple(t[60]) == (60, 4, 6)


# ---------------------------------------------------------------------------------------
# Small workloads: full comparison.
# ---------------------------------------------------------------------------------------
def test_workload_512_full():
    _, M, N, K, dist, seed = workload("gemm512_u")
    A, B = operands(M, N, K, dist, seed)
    C = from_dev(run(to_dev(A), to_dev(B), M, N, K))
    want = oracle.gemm(A, B)
    assert_within_tolerance(C, want, "512^3")
    # the tutorial's own check: allclose against torch.matmul with atol 1e-2, rtol 0
    ref = torch.matmul(to_dev(A).view(torch.float16), to_dev(B).view(torch.float16))
    got = torch.from_numpy(C.view(np.float16)).cuda()
    assert torch.allclose(got, ref, atol=1e-2, rtol=0)


def test_workload_1024x768x128_grouped_full():
    _, M, N, K, dist, seed = workload("gemm1024x768x128_u01")
    A, B = operands(M, N, K, dist, seed)
    opts = dict(tile=g.TILE_128x64x64, group_m=2)
    rc, info = g.gemm_f16f32_plan(M, N, K, 1 << 20, 2 << 20, 3 << 20, K, N, N, opts=opts)
    assert rc == g.OK and (info["num_pid_m"], info["num_pid_n"]) == (8, 12)
    C = from_dev(run(to_dev(A), to_dev(B), M, N, K, **opts))
    assert_within_tolerance(C, oracle.gemm(A, B), "1024x768x128")
    for remap in (g.REMAP_ON, g.REMAP_OFF):
        got = g.tile_map(8, 12, 2, remap).cpu().numpy().astype(np.int64)
        assert np.array_equal(got, oracle.program_tiles(8, 12, 2, remap == g.REMAP_ON))


# ---------------------------------------------------------------------------------------
# Full-size workloads: every element of C against the oracle.
# ---------------------------------------------------------------------------------------
_ORACLE_CACHE = {}


def full_oracle(name):
    """Operands and the oracle's whole C for a named workload (computed once per session)."""
    if name not in _ORACLE_CACHE:
        _, M, N, K, dist, seed = workload(name)
        A, B = operands(M, N, K, dist, seed)
        print(f"oracle {name}: {M}x{N}x{K} on {oracle.num_threads()} threads", flush=True)
        _ORACLE_CACHE[name] = (A, B, oracle.gemm(A, B))
    return _ORACLE_CACHE[name]


@pytest.mark.parametrize("name,opts", [
    ("gemm4096_u", {}),
    ("gemm8192_u", {}),
    ("gemm4095x4097x4093_n", {"group_m": 6}),   # 16 x 17 tiles: last group of 4 tile rows
    ("gemm4095x4097x4093_n", {}),               # the library's own plan
])
def test_large_workload_every_element(name, opts):
    """The launch configuration the benchmark times (the library's plan, or G = 6 for the
    ragged shape's partial last group), compared with the oracle at every element of C."""
    _, M, N, K, dist, seed = workload(name)
    A, B, want = full_oracle(name)
    rc, info = g.gemm_f16f32_plan(M, N, K, 1 << 40, 2 << 40, 3 << 40, K, N, N,
                                  opts=opts or None)
    assert rc == g.OK
    if opts.get("group_m") == 6:
        assert info["num_pid_m"] % 6 == 4
    print(f"gpu {name} {opts}: tile {info['tile']} G {info['group_m']} "
          f"launches {info['launches']}", flush=True)
    Cd = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda")   # NaN until written
    C = from_dev(run(to_dev(A), to_dev(B), M, N, K, C_dev=Cd, **opts))
    assert_within_tolerance(C, want, f"{name} {opts}")
    assert checksum_ok(A, B, C), name


def test_8192_run_to_run_bit_identical():
    """Two launches of the benchmark's configuration at 8192^3 give the same bits: every
    element's fp32 sum is formed in one fixed order, whatever the timing of the panel
    pipeline or of the other workgroups."""
    _, M, N, K, dist, seed = workload("gemm8192_u")
    A, B, want = full_oracle("gemm8192_u")
    Ad, Bd = to_dev(A), to_dev(B)
    first = from_dev(run(Ad, Bd, M, N, K))
    torch.cuda.synchronize()
    Cd = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda")
    second = from_dev(run(Ad, Bd, M, N, K, C_dev=Cd))
    assert np.array_equal(first, second)
    assert_within_tolerance(second, want, "8192^3 second launch")


@pytest.mark.parametrize("tile", [g.TILE_256x256x64, g.TILE_256x256x32])
def test_ragged_equals_front_padded(tile):
    """The ragged run equals, bit for bit, a run on operands zero-padded to tile multiples:
    in front of k (the DMA path puts the K mod BK leading k values at the end of its first
    panel), after the last row of A and after the last column of B.  Zeros add +0 to the same
    fp32 sums in the same order."""
    _, M, N, K, dist, seed = workload("gemm4095x4097x4093_n")
    A, B = operands(M, N, K, dist, seed)
    bk = 64 if tile == g.TILE_256x256x64 else 32
    pad = (-K) % bk
    Mp, Np, Kp = 4096, 4104, K + pad
    Ap = np.zeros((Mp, Kp), np.uint16)
    Ap[:M, pad:] = A
    Bp = np.zeros((Kp, Np), np.uint16)
    Bp[pad:, :N] = B
    opts = dict(tile=tile, group_m=6)
    C = from_dev(run(to_dev(A), to_dev(B), M, N, K, **opts))
    Cp = from_dev(run(to_dev(Ap), to_dev(Bp), Mp, Np, Kp, **opts))
    assert np.array_equal(C, Cp[:M, :N])


@pytest.mark.parametrize("M,N", [(4095, 4097), (4096 + 3, 4096 + 5), (4096 + 64, 4096 + 1)])
def test_edge_split_changes_no_bit(M, N):
    """Splitting thin edge slivers into their own launches leaves every element unchanged."""
    K = 1000
    A, B = operands(M, N, K, "n(0,0.1)", M + N)
    Ad, Bd = to_dev(A), to_dev(B)
    rc, info = g.gemm_f16f32_plan(M, N, K, 1 << 40, 2 << 40, 3 << 40, K, N, N)
    assert info["launches"] > 1 or info["strip_n"] > 0   # split off, or taken into the launch
    split = from_dev(run(Ad, Bd, M, N, K))
    whole = from_dev(run(Ad, Bd, M, N, K, split_edges=g.SPLIT_OFF))
    assert np.array_equal(split, whole)
    assert_within_tolerance(split, oracle.gemm(A, B), f"{M}x{N} split")


def test_ragged_generic_path_within_tolerance():
    """The register-staged generic path on the ragged shape (its own k order)."""
    _, M, N, K, dist, seed = workload("gemm4095x4097x4093_n")
    A, B, want = full_oracle("gemm4095x4097x4093_n")
    C = from_dev(run(to_dev(A), to_dev(B), M, N, K, force_generic=1, group_m=6))
    assert_within_tolerance(C, want, "generic ragged")


# ---------------------------------------------------------------------------------------
# Invariants on one shape: paths, alignment, group size and remap change no bit.
# ---------------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def ops2048():
    A, B = operands(2048, 2048, 2048, "u(-0.5,0.5)", 7)
    return A, B, to_dev(A), to_dev(B)


def test_paths_and_alignment_change_no_bit(ops2048):
    """With 64-deep panels and K a multiple of 64 the DMA and generic paths add the same
    products in the same order, so they agree bit for bit -- also on operands that start 2 or
    6 bytes past an aligned address (rows only 2-byte aligned)."""
    A, B, Ad, Bd = ops2048
    ref = from_dev(run(Ad, Bd, 2048, 2048, 2048, tile=g.TILE_256x256x64))
    gen = from_dev(run(Ad, Bd, 2048, 2048, 2048, tile=g.TILE_256x256x64, force_generic=1))
    assert np.array_equal(ref, gen)
    Ab = torch.zeros(2048 * 2048 + 8, dtype=torch.int16, device="cuda")
    Bb = torch.zeros(2048 * 2048 + 8, dtype=torch.int16, device="cuda")
    Ab[1:1 + 2048 * 2048] = Ad.reshape(-1)
    Bb[3:3 + 2048 * 2048] = Bd.reshape(-1)
    Au = Ab[1:1 + 2048 * 2048].view(2048, 2048)
    Bu = Bb[3:3 + 2048 * 2048].view(2048, 2048)
    for fg in (0, 1):
        odd = from_dev(run(Au, Bu, 2048, 2048, 2048, tile=g.TILE_256x256x64, force_generic=fg))
        assert np.array_equal(ref, odd), fg


def test_group_and_remap_change_no_bit(ops2048):
    A, B, Ad, Bd = ops2048
    ref = from_dev(run(Ad, Bd, 2048, 2048, 2048, tile=g.TILE_256x256x64, group_m=1))
    for G in (2, 4, 8, 16):
        for remap in (g.REMAP_ON, g.REMAP_OFF):
            got = from_dev(run(Ad, Bd, 2048, 2048, 2048, tile=g.TILE_256x256x64, group_m=G,
                               xcd_remap=remap))
            assert np.array_equal(ref, got), (G, remap)


def test_run_to_run_deterministic(ops2048):
    A, B, Ad, Bd = ops2048
    first = from_dev(run(Ad, Bd, 2048, 2048, 2048))
    for _ in range(3):
        assert np.array_equal(first, from_dev(run(Ad, Bd, 2048, 2048, 2048)))


def test_every_tile_config_within_tolerance(ops2048):
    A, B, Ad, Bd = ops2048
    rows, cols = sample_positions(2048, 2048, 128, 128, 4, 1)
    want = oracle.gemm_sampled(A, B, rows, cols)
    for tile in g.TILES:
        for fg in (0, 1):
            C = from_dev(run(Ad, Bd, 2048, 2048, 2048, tile=tile, force_generic=fg))
            assert_within_tolerance(C[rows, cols], want, f"tile {tile} generic {fg}")


# ---------------------------------------------------------------------------------------
# Edge shapes against the full oracle, with canaries in the leading-dimension padding.
# ---------------------------------------------------------------------------------------
EDGE = [(1, 1, 1), (1, 1, 64), (7, 9, 13), (255, 1, 61), (257, 129, 65), (300, 200, 64),
        (64, 64, 4096), (33, 8, 64), (129, 65, 127), (511, 513, 190), (2, 300, 1), (256, 256, 64)]


@pytest.mark.parametrize("M,N,K", EDGE)
@pytest.mark.parametrize("tile", sorted(g.TILES))
def test_edge_shapes_full_oracle(M, N, K, tile):
    A, B = operands(M, N, K, "n(0,0.1)", M * 7 + N * 3 + K)
    pad = 3
    ldc = N + pad
    Cd = torch.full((M, ldc), 0x5A5A, dtype=torch.int16, device="cuda")
    run(to_dev(A), to_dev(B), M, N, K, C_dev=Cd, tile=tile)
    C = from_dev(Cd)
    assert_within_tolerance(C[:, :N], oracle.gemm(A, B), f"{M}x{N}x{K} tile {tile}")
    assert np.all(C[:, N:] == 0x5A5A), "wrote into the ldc padding"


@pytest.mark.parametrize("lda_pad,ldb_pad", [(1, 0), (0, 1), (5, 3), (8, 8)])
def test_leading_dimensions(lda_pad, ldb_pad):
    M, N, K = 300, 264, 192
    A, B = operands(M, N, K, "u(-0.5,0.5)", 5)
    Ap = np.full((M, K + lda_pad), 0x7C00, np.uint16)  # +inf in the padding: must not be read
    Ap[:, :K] = A
    Bp = np.full((K, N + ldb_pad), 0x7C00, np.uint16)
    Bp[:, :N] = B
    C = from_dev(run(to_dev(Ap), to_dev(Bp), M, N, K))
    assert_within_tolerance(C, oracle.gemm(A, B), f"lda pad {lda_pad}, ldb pad {ldb_pad}")


def test_k_zero_writes_positive_zero():
    Cd = torch.full((5, 7), 0x1234, dtype=torch.int16, device="cuda")
    Ad = torch.zeros((5, 1), dtype=torch.int16, device="cuda")
    Bd = torch.zeros((1, 7), dtype=torch.int16, device="cuda")
    run(Ad, Bd, 5, 7, 0, C_dev=Cd)
    assert np.all(from_dev(Cd) == 0)


# ---------------------------------------------------------------------------------------
# Closed forms that are exact in fp32, so every correct kernel gives the same bits.
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("K,want", [(2048, 2048.0), (2051, 2052.0), (4093, 4092.0),
                                    (4095, 4096.0), (4096, 4096.0)])
def test_all_ones_round_half_even(K, want):
    """K ones sum to K exactly in fp32; above 2048 the fp16 spacing is 2 and odd K are ties
    that round to the even pattern (round toward zero would give K - 1)."""
    M, N = 256, 264
    one = np.float16(1.0).view(np.uint16)
    A = np.full((M, K), one, np.uint16)
    B = np.full((K, N), one, np.uint16)
    C = from_dev(run(to_dev(A), to_dev(B), M, N, K))
    assert np.all(C == np.float16(want).view(np.uint16))


def test_identity_gives_b_exactly():
    K, N = 384, 256
    A = np.eye(K, dtype=np.float16).view(np.uint16)
    _, B = operands(1, N, K, "n(0,0.1)", 3)
    C = from_dev(run(to_dev(A), to_dev(B), K, N, K))
    assert np.array_equal(C, B)


def test_one_hot_last_k_selects_last_row_of_b():
    M, N, K = 320, 272, 4093
    A = np.zeros((M, K), np.uint16)
    A[:, K - 1] = np.float16(1.0).view(np.uint16)
    _, B = operands(1, N, K, "u(-0.5,0.5)", 9)
    C = from_dev(run(to_dev(A), to_dev(B), M, N, K))
    assert np.array_equal(C, np.broadcast_to(B[K - 1], (M, N)))


def test_graph_capture_replays_match_eager():
    """The library launches on the caller's stream, so a HIP graph captured around calls
    replays them; every replay (with eager work in between) must match the eager result."""
    M, N, K = 1000, 1100, 900
    A, B = operands(M, N, K, "u(-0.5,0.5)", 21)
    Ad, Bd = to_dev(A), to_dev(B)
    eager = from_dev(run(Ad, Bd, M, N, K))
    Cg = torch.zeros((M, N), dtype=torch.int16, device="cuda")
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(Ad, Bd, M, N, K, C_dev=Cg)          # warm-up on the side stream
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(graph):
        run(Ad, Bd, M, N, K, C_dev=Cg)
    for rep in range(3):
        Cg.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(from_dev(Cg), eager), rep
        other = from_dev(run(Ad, Bd, 500, 600, K))   # unrelated eager work in between
        assert_within_tolerance(other, eager[:500, :600], "eager between replays")


@pytest.mark.parametrize("M,N,K,tile", [
    (2048, 2048, 2048, g.TILE_256x256x64),          # fewer programs than the grid
    (8192, 4096, 512, g.TILE_256x256x64),           # 512 programs on 256 workgroups
    (8192, 4096, 512, g.TILE_256x256x64_W8),
    (2048, 2048, 1000, g.TILE_64x64x64),            # 1024 programs on 512 workgroups
    (3000, 1000, 700, g.TILE_32x32x64),             # 2976 programs, ragged, 5 per CU
    (4095, 4097, 4093, 0),                          # library's choice, with the edge split
])
def test_persistent_schedule_changes_no_bit(M, N, K, tile):
    """Workgroup h of the persistent grid computes programs h, h + grid, ...: every tile once,
    with the same k order, so the result equals the one-workgroup-per-program launch."""
    A, B = operands(M, N, K, "u(-0.5,0.5)", M + N + K)
    Ad, Bd = to_dev(A), to_dev(B)
    opts = dict(tile=tile) if tile else {}
    rc, info = g.gemm_f16f32_plan(M, N, K, 1 << 40, 2 << 40, 3 << 40, K, N, N,
                                  opts=dict(opts, persistent=g.PERSISTENT_ON))
    assert rc == g.OK and info["persistent"] == 1 and info["grid"] <= info["num_programs"]
    Cd = torch.full((M, N), 0x7E00, dtype=torch.int16, device="cuda")
    plain = from_dev(run(Ad, Bd, M, N, K, **opts))
    pers = from_dev(run(Ad, Bd, M, N, K, C_dev=Cd, persistent=g.PERSISTENT_ON, **opts))
    assert np.array_equal(plain, pers)
    assert_within_tolerance(pers, oracle.gemm(A, B), f"{M}x{N}x{K}")


# The 256 x 256 x 64 kernels (one workgroup per program, persistent, split K) keep their
# panels in five LDS slots whose indices repeat every 6 panels (A in a ring of three, B in a
# ring of two), and leave their unrolled loop after the last panel.  The panel counts below end
# at every position of the unrolled loop, with and without a head panel (K not a multiple of
# 64), with a ragged last tile row and column, and with the operands' last element patched in
# the last panel (odd leading dimensions); the split K slices start and end at other panels.
# The 256 x 256 x 32 tile (four LDS stages, 32x32x16 MFMAs) gives the same bits.
@pytest.mark.parametrize("K", [64, 128, 192, 256, 320, 384, 448, 768, 832, 17, 64 * 6 + 1,
                               64 * 7 + 63, 64 * 12 + 5])
@pytest.mark.parametrize("M,N,pad", [(512, 512, 0), (300, 520, 0), (513, 257, 1)])
def test_five_slot_schedule_matches_the_staged_tile(M, N, K, pad):
    print(f"five-slot schedule {M}x{N}x{K} pad {pad}", flush=True)
    A, B = operands(M, N, K, "n(0,0.1)", M + 3 * N + 7 * K)
    Ad, Bd = to_dev(A), to_dev(B)
    if pad:
        Ap = torch.zeros((M, K + pad), dtype=torch.int16, device="cuda")
        Bp = torch.zeros((K, N + pad), dtype=torch.int16, device="cuda")
        Ap[:, :K] = Ad
        Bp[:, :N] = Bd
        Ad, Bd = Ap[:, :K], Bp[:, :N]
    ring, staged = g.TILE_256x256x64, g.TILE_256x256x32
    want = from_dev(g.matmul(Ad, Bd, tile=staged))
    got = from_dev(g.matmul(Ad, Bd, tile=ring))
    pers = from_dev(g.matmul(Ad, Bd, tile=ring, persistent=g.PERSISTENT_ON))
    assert np.array_equal(got, want)
    assert np.array_equal(pers, want)
    ref = oracle.gemm(A, B)
    assert_within_tolerance(got, ref, f"{M}x{N}x{K}")
    for S in (2, 3):
        split = from_dev(g.matmul(Ad, Bd, tile=ring, split_k=S))
        assert np.array_equal(split, from_dev(g.matmul(Ad, Bd, tile=staged, split_k=S))), S
        assert_within_tolerance(split, ref, f"{M}x{N}x{K} split {S}")
