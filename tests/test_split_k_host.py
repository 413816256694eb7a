"""Host-side checks of split K (opts.split_k, gemm_f16f32_strided_ws) that need no GPU.

The plan's slice count, slice depth, workspace size and grid follow the documented rule
(L = roundup(cdiv(K, S), 128), S' = cdiv(K, L), workspace S' M roundup(N, 4) 4 bytes), the
slices do not depend on the tile, and every misuse is rejected with its documented code
before anything is launched.  No call here launches a kernel.
"""
import pytest

import dense_gemm_f16f32_amd as g

# Fake, never dereferenced device addresses (16-byte aligned, far apart).
PA, PB, PC, PW = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def cdiv(x, y):
    return -(-x // y)


def plan(M, N, K, **opts):
    rc, info = g.gemm_f16f32_strided_plan(M, N, K, PA, K, 1, PB, N, 1, PC, N, 1, opts=opts)
    assert rc == g.OK, g.gemm_f16f32_strerror(rc)
    return info


def ws_call(M, N, K, ws, nbytes, **opts):
    return g.gemm_f16f32_strided_ws(M, N, K, PA, K, 1, PB, N, 1, PC, N, 1, ws, nbytes, None,
                                    opts)


@pytest.mark.parametrize("M,N,K,S", [(256, 256, 8192, 4), (64, 64, 1000, 3), (100, 37, 4093, 7),
                                     (1, 1, 640, 5), (2048, 2048, 8192, 16), (33, 1, 129, 2)])
def test_split_plan_follows_the_rule(M, N, K, S):
    info = plan(M, N, K, split_k=S)
    L = cdiv(cdiv(K, S), 128) * 128
    want_s = cdiv(K, L)
    assert want_s >= 2
    assert info["splits"] == want_s and info["split_depth"] == L
    assert info["workspace_bytes"] == want_s * M * (cdiv(N, 4) * 4) * 4
    assert info["grid"] == want_s * info["num_programs"]
    assert info["launches"] == 2 and info["persistent"] == 0
    assert info["main_m"] == M and info["main_n"] == N   # no edge split
    # the first slice holds what is left in front: 1 .. L k values
    assert 1 <= K - (want_s - 1) * L <= L


@pytest.mark.parametrize("K,S", [(0, 4), (100, 2), (128, 8), (128, 2), (64, 3)])
def test_no_split_when_k_fits_one_slice(K, S):
    info = plan(96, 80, K, split_k=S)
    assert info["splits"] == 1 and info["split_depth"] == 0 and info["workspace_bytes"] == 0
    # ... and then the entry points without a workspace accept the option
    assert g.gemm_f16f32_strided_ws(0, 80, K, PA, max(K, 1), 1, PB, 80, 1, PC, 80, 1, 0, 0,
                                    None, dict(split_k=S)) == g.OK


@pytest.mark.parametrize("S", [0, 1])
def test_split_k_zero_and_one_mean_off(S):
    info = plan(128, 128, 8192, split_k=S)
    assert info["splits"] == 1 and info["workspace_bytes"] == 0


def test_slices_do_not_depend_on_the_tile():
    M, N, K, S = 200, 150, 1500, 3
    seen = set()
    for t in sorted(g.TILES):
        info = plan(M, N, K, split_k=S, tile=t)
        assert info["tile"] == t and info["bk"] == g.TILES[t][2]
        assert info["split_depth"] % info["bk"] == 0
        seen.add((info["splits"], info["split_depth"], info["workspace_bytes"]))
    assert seen == {(3, 512, 3 * 200 * 152 * 4)}


def test_split_tile_is_chosen_for_the_slice_shape():
    # the planner picks the tile for M x N x L, the shape each slice computes
    M, N, K, S = 512, 512, 8192, 8
    split = plan(M, N, K, split_k=S)
    L = split["split_depth"]
    sliced = plan(M, N, L, split_edges=g.SPLIT_OFF)
    assert split["tile"] == sliced["tile"]


def test_column_major_c_plans_the_transpose():
    M, N, K = 100, 30, 2000
    rc, info = g.gemm_f16f32_strided_plan(M, N, K, PA, K, 1, PB, N, 1, PC, 1, M,
                                          opts=dict(split_k=4))
    assert rc == g.OK and info["swapped"] == 1
    assert info["workspace_bytes"] == info["splits"] * N * (cdiv(M, 4) * 4) * 4


def test_option_errors():
    for bad in (dict(split_k=-2), dict(split_k=2, force_generic=1),
                dict(split_k=4, persistent=g.PERSISTENT_ON)):
        rc, _ = g.gemm_f16f32_strided_plan(64, 64, 4096, PA, 4096, 1, PB, 64, 1, PC, 64, 1,
                                           opts=bad)
        assert rc == g.ERR_OPTS, bad
    # persistent "off" and the generic path "off" are fine
    assert plan(64, 64, 4096, split_k=4, persistent=g.PERSISTENT_OFF, force_generic=0)[
        "splits"] == 4


def test_entry_points_without_a_workspace_refuse_a_split():
    o = g.Opts(split_k=4)
    assert g.gemm_f16f32_ex(64, 64, 4096, PA, PB, PC, 4096, 64, 64, None, o) == g.ERR_WORKSPACE
    assert g.gemm_f16f32_strided(64, 64, 4096, PA, 4096, 1, PB, 64, 1, PC, 64, 1, None,
                                 o) == g.ERR_WORKSPACE


def test_workspace_errors():
    M, N, K = 64, 64, 4096
    need = plan(M, N, K, split_k=4)["workspace_bytes"]
    assert need == 4 * 64 * 64 * 4
    assert ws_call(M, N, K, 0, need, split_k=4) == g.ERR_WORKSPACE           # NULL
    assert ws_call(M, N, K, PW, need - 1, split_k=4) == g.ERR_WORKSPACE      # too small
    assert ws_call(M, N, K, PW + 8, need, split_k=4) == g.ERR_WORKSPACE      # not 16-aligned
    assert ws_call(M, N, K, PC - need + 16, need, split_k=4) == g.ERR_OVERLAP  # into C
    assert ws_call(M, N, K, PA + 64, need, split_k=4) == g.ERR_OVERLAP       # inside A
    assert ws_call(M, N, K, PB - 16, need, split_k=4) == g.ERR_OVERLAP       # into B
    # argument errors come first, as in the other entry points
    assert ws_call(-1, N, K, PW, need, split_k=4) == g.ERR_DIM


def test_workspace_offsets_too_large():
    # 256 rows of a 2^22-wide fp32 workspace are 2^32 bytes: beyond 32-bit offsets
    M, N, K = 256, 1 << 22, 8192
    rc, _ = g.gemm_f16f32_strided_plan(M, N, K, PA, K, 1, 1 << 40, N, 1, 2 << 40, N, 1,
                                       opts=dict(split_k=2, tile=g.TILE_256x256x64))
    assert rc == g.ERR_TOO_LARGE
    rc, _ = g.gemm_f16f32_strided_plan(M, N, K, PA, K, 1, 1 << 40, N, 1, 2 << 40, N, 1,
                                       opts=dict(tile=g.TILE_256x256x64))
    assert rc == g.OK


def test_strerror_names_the_workspace():
    assert "workspace" in g.gemm_f16f32_strerror(g.ERR_WORKSPACE)


def auto_rule(M, N, K):
    """The documented automatic choice: the largest power of two S <= 16 with K >= 512 S whose
    split grid (S times the programs of the tile planned for M x N x L) fits in 256 CUs;
    S = 2 only from K = 4096 on."""
    best, S = 1, 2
    while S <= 16 and K >= 512 * S:
        L = cdiv(cdiv(K, S), 128) * 128
        if plan(M, N, L, split_edges=g.SPLIT_OFF)["num_programs"] * S <= 256:
            best = S
        S *= 2
    return 1 if (best == 2 and K < 4096) else best


@pytest.mark.parametrize("M,N,K", [(32, 32, 8192), (32, 32, 1024), (64, 64, 2048),
                                   (256, 256, 4096), (512, 512, 8192), (512, 512, 2048),
                                   (2048, 2048, 8192), (4095, 1, 4093), (1, 1, 65536),
                                   (64, 4096, 8192), (100, 100, 0)])
def test_automatic_split_follows_the_rule(M, N, K):
    info = plan(M, N, K, split_k=g.SPLIT_K_AUTO)
    S = auto_rule(M, N, K) if K > 0 else 1
    if S == 1:
        assert info["splits"] == 1 and info["workspace_bytes"] == 0
    else:
        L = cdiv(cdiv(K, S), 128) * 128
        assert info["splits"] == cdiv(K, L) and info["split_depth"] == L
        assert info == plan(M, N, K, split_k=S)


def test_automatic_split_cases():
    # thin, deep problems split; large or shallow ones do not
    assert plan(32, 32, 8192, split_k=g.SPLIT_K_AUTO)["splits"] == 16
    assert plan(64, 64, 1024, split_k=g.SPLIT_K_AUTO)["splits"] == 1
    assert plan(2048, 2048, 8192, split_k=g.SPLIT_K_AUTO)["splits"] == 1
    # automatic mode never errors for options that exclude a split; it just does not split
    for o in (dict(force_generic=1), dict(persistent=g.PERSISTENT_ON)):
        assert plan(32, 32, 8192, split_k=g.SPLIT_K_AUTO, **o)["splits"] == 1
    rc, _ = g.gemm_f16f32_strided_plan(64, 64, 4096, PA, 4096, 1, PB, 64, 1, PC, 64, 1,
                                       opts=dict(split_k=-2))
    assert rc == g.ERR_OPTS
