"""Host-side checks of libgemm_f16f32.so that need no GPU.

The library loads, exports every function include/gemm_f16f32.h declares, rejects bad
arguments with the documented codes before touching the GPU, and plans the documented kernel
path, tile, GROUP_SIZE_M and grid.  No call here launches a kernel.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import dense_gemm_f16f32_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gemm_f16f32.h")

# Fake, never dereferenced device addresses (16-byte aligned, far apart).
PA, PB, PC = 0x10000000, 0x20000000, 0x30000000


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_f16f32\w*)\s*\(", text)))


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert "gemm_f16f32" in names and "gemm_f16f32_tile_map" in names
    L = ctypes.CDLL(g.LIB_PATH)
    for n in names:
        assert hasattr(L, n), n


def test_version_and_strerror():
    assert g.gemm_f16f32_version() >= 100
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9]:
        assert g.gemm_f16f32_strerror(code) and g.gemm_f16f32_strerror(code) != "unknown error code"
    assert g.gemm_f16f32_strerror(-99) == "unknown error code"


@pytest.mark.parametrize("args,code", [
    ((-1, 8, 8, PA, PB, PC, 8, 8, 8), g.ERR_DIM),
    ((8, -1, 8, PA, PB, PC, 8, 8, 8), g.ERR_DIM),
    ((8, 8, -1, PA, PB, PC, 8, 8, 8), g.ERR_DIM),
    ((1 << 31, 8, 8, PA, PB, PC, 8, 8, 8), g.ERR_DIM),
    ((8, 8, 8, PA, PB, PC, 7, 8, 8), g.ERR_LD),
    ((8, 8, 8, PA, PB, PC, 8, 7, 8), g.ERR_LD),
    ((8, 8, 8, PA, PB, PC, 8, 8, 7), g.ERR_LD),
    ((8, 8, 0, PA, PB, PC, 0, 8, 8), g.ERR_LD),
    ((8, 8, 8, 0, PB, PC, 8, 8, 8), g.ERR_NULL),
    ((8, 8, 8, PA, 0, PC, 8, 8, 8), g.ERR_NULL),
    ((8, 8, 8, PA, PB, 0, 8, 8, 8), g.ERR_NULL),
    ((8, 8, 8, PA, PB, PA + 16, 8, 8, 8), g.ERR_OVERLAP),
    ((8, 8, 8, PA, PB, PB + 126, 8, 8, 8), g.ERR_OVERLAP),
    ((8, 8, 8, PA + 1, PB, PC, 8, 8, 8), g.ERR_OPTS),
    ((8, 8, 8, 1 << 40, 2 << 40, 3 << 40, 1 << 26, 8, 8), g.ERR_TOO_LARGE),  # 64 x lda >= 2^31
])
def test_argument_errors_before_launch(args, code):
    assert g.gemm_f16f32(*args, None) == code
    rc, _ = g.gemm_f16f32_plan(*args)
    assert rc == code


def test_empty_problems_are_noops():
    # M == 0 or N == 0: success without any GPU call (no device here), NULL pointers allowed.
    assert g.gemm_f16f32(0, 8, 8, 0, 0, 0, 8, 8, 8, None) == g.OK
    assert g.gemm_f16f32(8, 0, 8, 0, 0, 0, 8, 1, 1, None) == g.OK
    rc, info = g.gemm_f16f32_plan(0, 8, 8, 0, 0, 0, 8, 8, 8)
    assert rc == g.OK and info["num_programs"] == 0
    # K == 0 needs C only
    rc, info = g.gemm_f16f32_plan(8, 8, 0, 0, 0, PC, 1, 8, 8)
    assert rc == g.OK and info["num_programs"] > 0


def test_option_errors():
    base = (64, 64, 64, PA, PB, PC, 64, 64, 64)
    for bad in ({"tile": max(g.TILES) + 1}, {"tile": -1}, {"group_m": -1}, {"xcd_remap": 3}, {"force_generic": 2},
                {"split_edges": 3}):
        assert g.gemm_f16f32_plan(*base, opts=bad)[0] == g.ERR_OPTS
        assert g.gemm_f16f32_ex(*base, None, bad) == g.ERR_OPTS


def test_tile_map_argument_errors():
    assert g.gemm_f16f32_tile_map(0, 4, 1, 0, PC) == g.ERR_DIM
    assert g.gemm_f16f32_tile_map(4, 4, 0, 0, PC) == g.ERR_OPTS
    assert g.gemm_f16f32_tile_map(4, 4, 1, 3, PC) == g.ERR_OPTS
    assert g.gemm_f16f32_tile_map(4, 4, 1, 0, 0) == g.ERR_NULL
    assert g.gemm_f16f32_tile_map(1 << 16, 1 << 16, 1, 0, PC) == g.ERR_DIM


def plan(M, N, K, lda=None, ldb=None, ldc=None, a=PA, b=PB, c=PC, **opts):
    rc, info = g.gemm_f16f32_plan(M, N, K, a, b, c, lda or K, ldb or N, ldc or N,
                                  opts=opts or None)
    assert rc == g.OK
    return info


TUNE_TABLE = os.path.join(ROOT, "dense_gemm_f16f32_amd", "csrc", "tune_table.inc")


def tune_entries():
    """(log2 M, log2 N, log2 K) -> (tile, group, remap) rows of the compiled dispatch table."""
    rows = {}
    for ln in open(TUNE_TABLE):
        m = re.match(r"\s*\{(-?\d+), (-?\d+), (-?\d+), (\d+), (\d+), (\d+)\}", ln)
        if m:
            lm, lnn, lk, tile, grp, remap = map(int, m.groups())
            rows[(lm, lnn, lk)] = (tile, grp, remap)
    return rows


def shape_class(M, N, K):
    def c(x, lo, hi):
        return min(max(lo if x < 1 else int(round(np.log2(x))), lo), hi)
    return c(M, 5, 13), c(N, 5, 13), c(K, 6, 13)


def expected_choice(M, N, K):
    """The table's (tile, group) for this shape class, or None (heuristic)."""
    return tune_entries().get(shape_class(M, N, K))


def test_tune_table_rows_are_valid():
    rows = tune_entries()
    assert len(rows) == 9 * 9 * 8
    for key, (tile, grp, remap) in rows.items():
        assert tile in g.TILES and 0 <= grp <= 64 and remap in (0, 2), key
        assert 5 <= key[0] <= 13 and 5 <= key[1] <= 13 and 6 <= key[2] <= 13, key


def test_planner_follows_the_table():
    for (lm, ln, lk), (tile, grp, remap) in sorted(tune_entries().items()):
        M, N, K = 1 << lm, 1 << ln, 1 << lk
        p = plan(M, N, K)
        assert p["tile"] == tile, (M, N, K)
        want_g = grp or plan(M, N, K, tile=tile)["group_m"]
        assert p["group_m"] == want_g, (M, N, K)
        assert p["xcd_remap"] == (0 if remap == 2 else 1), (M, N, K)
        # a non-power-of-two shape in the same class gets the same tile
        p2 = plan(M + M // 8, N, K)
        if shape_class(M + M // 8, N, K) == (lm, ln, lk) and p2["launches"] == 1:
            assert p2["tile"] == tile


def test_plans_for_the_five_workloads():
    for M, N, K in [(512, 512, 512), (4096, 4096, 4096), (8192, 8192, 8192)]:
        p = plan(M, N, K)
        bm, bn = g.TILES[p["tile"]][:2]
        assert p["path"] == g.PATH_DMA and (p["bm"], p["bn"]) == (bm, bn)
        assert p["num_programs"] == -(-M // bm) * -(-N // bn)
        want = expected_choice(M, N, K)
        if want:
            assert p["tile"] == want[0]
    # the pages' worked example, forced: 128 x 64 tiles with G = 2
    p = plan(1024, 768, 128, tile=g.TILE_128x64x64, group_m=2)
    assert (p["num_pid_m"], p["num_pid_n"], p["num_programs"], p["group_m"]) == (8, 12, 96, 2)
    # 8192^3 follows the table's order (measured: G = 2 with the XCD permutation off); an
    # explicit option overrides it
    want = tune_entries()[shape_class(8192, 8192, 8192)]
    p = plan(8192, 8192, 8192)
    assert (p["group_m"] if want[1] else 0, p["xcd_remap"]) == (want[1], 0 if want[2] == 2 else 1)
    assert plan(8192, 8192, 8192, xcd_remap=g.REMAP_ON)["xcd_remap"] == 1
    assert plan(8192, 8192, 8192, xcd_remap=g.REMAP_OFF)["xcd_remap"] == 0
    # ragged, 256 x 256 tiles: the 1-column sliver is split off, the main launch covers
    # 4095 x 4096 with 16 x 16 tiles
    p = plan(4095, 4097, 4093, tile=g.TILE_256x256x64, group_m=6, split_edges=g.SPLIT_ON)
    assert (p["path"], p["num_pid_m"], p["num_pid_n"], p["num_programs"]) == \
        (g.PATH_DMA, 16, 16, 256)
    assert (p["launches"], p["main_m"], p["main_n"]) == (2, 4095, 4096)
    p = plan(4095, 4097, 4093, tile=g.TILE_256x256x64, group_m=6)
    assert (p["num_pid_m"], p["num_pid_n"], p["num_programs"], p["launches"]) == (16, 17, 272, 1)
    # the library's own plan: the ping-pong tile (odd leading dimensions) computes the
    # 1-column sliver inside its own launch
    p = plan(4095, 4097, 4093)
    assert p["tile"] == g.TILE_256x256x32_PP
    assert (p["launches"], p["main_n"], p["strip_n"], p["num_pid_n"]) == (1, 4096, 1, 16)
    # the same shape with aligned rows keeps the 256 x 256 x 64 tile and a second launch
    p = plan(4095, 4097, 4093, lda=4096, ldb=4104, ldc=4104)
    if p["tile"] == g.TILE_256x256x64:
        assert (p["launches"], p["main_n"], p["strip_n"]) == (2, 4096, 0)


def test_path_selection():
    """The DMA path takes every shape, leading dimension and 2-byte alignment; the generic
    path runs only when forced.  bk reports the panel depth of the kernel chosen."""
    for kw in ({}, {"K": 200}, {"N": 250, "ldb": 256, "ldc": 256}, {"lda": 260},
               {"a": PA + 2}, {"b": PB + 6, "ldb": 257}, {"M": 300}):
        args = dict(M=256, N=256, K=256)
        args.update(kw)
        M, N, K = args.pop("M"), args.pop("N"), args.pop("K")
        p = plan(M, N, K, **args)
        assert p["path"] == g.PATH_DMA and p["bk"] == 64, kw
    assert plan(256, 256, 96, tile=g.TILE_256x256x32)["bk"] == 32
    p = plan(256, 256, 256, force_generic=1)
    assert p["path"] == g.PATH_GENERIC and p["bk"] == 64
    assert plan(256, 256, 256, xcd_remap=2)["xcd_remap"] == 0


@pytest.mark.parametrize("M,N,want", [
    (4096, 4096, (1, 4096, 4096)),        # no remainder
    (4096, 4097, (2, 4096, 4096)),        # 1-column sliver
    (4096 + 64, 4096, (2, 4096, 4096)),   # 64-row sliver (<= 1/4 of 256)
    (4096 + 65, 4096, (1, 4161, 4096)),   # 65 rows: more than a quarter, kept
    (4096 + 3, 4096 + 5, (4, 4096, 4096)),  # right, bottom and corner strips
    (1000, 1001, (1, 1000, 1001)),        # small: fewer than 128 full tiles, kept
])
def test_edge_split_plans(M, N, want):
    """With 256 x 256 tiles: slivers of at most a quarter tile are split off."""
    p = plan(M, N, 512, tile=g.TILE_256x256x64, split_edges=g.SPLIT_ON)
    assert (p["launches"], p["main_m"], p["main_n"]) == want
    assert plan(M, N, 512, split_edges=g.SPLIT_OFF)["launches"] == 1
    # a forced tile splits only when asked
    assert plan(M, N, 512, tile=g.TILE_256x256x64)["launches"] == 1
    # a library-chosen tile splits by default, by the same rule for its own tile size
    p = plan(M, N, 512)
    bm, bn = p["bm"], p["bn"]
    rm, rn = M % bm, N % bn
    big = (M // bm) * (N // bn) >= 128
    want_split = big and ((0 < rn and 4 * rn <= bn) or (0 < rm and 4 * rm <= bm))
    assert (p["launches"] > 1) == want_split


# ---- strided entry points ------------------------------------------------------------------

def splan(M, N, K, sa, sb, sc, a=PA, b=PB, c=PC, **opts):
    return g.gemm_f16f32_strided_plan(M, N, K, a, sa[0], sa[1], b, sb[0], sb[1], c, sc[0],
                                      sc[1], opts=opts or None)


def test_strided_row_major_matches_plain_plan():
    M, N, K = 4096, 4096, 4096
    rc, p = splan(M, N, K, (K, 1), (N, 1), (N, 1))
    assert rc == g.OK
    assert p == plan(M, N, K)
    assert (p["a_kmajor"], p["b_kmajor"], p["swapped"]) == (1, 0, 0)


@pytest.mark.parametrize("a_col,b_col", [(0, 0), (0, 1), (1, 0), (1, 1)])
@pytest.mark.parametrize("c_col", [0, 1])
def test_strided_layouts(a_col, b_col, c_col):
    """Each storage order maps to the kernels' operand orders; a column-major C swaps roles."""
    M, N, K = 1000, 600, 300
    sa = (1, M + 8) if a_col else (K + 8, 1)
    sb = (1, K + 8) if b_col else (N + 8, 1)
    sc = (1, M + 8) if c_col else (N + 8, 1)
    rc, p = splan(M, N, K, sa, sb, sc)
    assert rc == g.OK
    if not c_col:
        assert (p["a_kmajor"], p["b_kmajor"], p["swapped"]) == (1 - a_col, b_col, 0)
        rows, cols = M, N
    else:
        # C^T = B^T A^T: first operand B^T is k-major iff B is column-major, A^T iff A is
        # row-major; the launch's rows run along N
        assert (p["a_kmajor"], p["b_kmajor"], p["swapped"]) == (b_col, 1 - a_col, 1)
        rows, cols = N, M
    # the main launch covers all rows (columns), or all but an edge sliver split off
    assert p["main_m"] in (rows, rows - rows % p["bm"])
    assert p["main_n"] in (cols, cols - cols % p["bn"])
    assert (p["num_pid_m"], p["num_pid_n"]) == (-(-p["main_m"] // p["bm"]),
                                                -(-p["main_n"] // p["bn"]))


@pytest.mark.parametrize("sa,sb,sc", [
    ((300, 2), (600, 1), (600, 1)),      # A: no unit stride
    ((300, 1), (1, 1), (600, 1)),        # B: row-major needs sbk >= N, column-major sbn >= K
    ((299, 1), (600, 1), (600, 1)),      # A: row stride below K
    ((1, 999), (600, 1), (600, 1)),      # A column-major: column stride below M
    ((300, 1), (600, 1), (600, -1)),     # C: negative stride
    ((300, 1), (600, 1), (0, 1)),        # C: zero row stride
])
def test_strided_errors(sa, sb, sc):
    assert splan(1000, 600, 300, sa, sb, sc)[0] == g.ERR_LD
    assert g.gemm_f16f32_strided(1000, 600, 300, PA, sa[0], sa[1], PB, sb[0], sb[1], PC,
                                 sc[0], sc[1], None) == g.ERR_LD


def test_strided_degenerate_axes():
    # a stride along an axis of extent 1 is never used
    assert splan(1, 600, 300, (12345, 1), (600, 1), (7, 1))[0] == g.OK
    assert splan(1000, 1, 300, (300, 1), (1, 999), (1, 55))[0] == g.OK
    assert splan(1000, 600, 1, (1, 3), (600, 1), (600, 1))[0] == g.OK
    # empty matrices may have any strides; M == 0 launches nothing
    rc, p = splan(0, 600, 300, (0, 0), (600, 1), (0, 0))
    assert rc == g.OK and p["num_programs"] == 0
    rc, p = splan(8, 8, 0, (0, 0), (0, 0), (8, 1), a=0, b=0)
    assert rc == g.OK and p["num_programs"] > 0
    assert g.gemm_f16f32_strided(-1, 8, 8, PA, 8, 1, PB, 8, 1, PC, 8, 1, None) == g.ERR_DIM


def test_strided_overlap_uses_the_storage_footprint():
    # A column-major (K x M in memory): footprint 2((K-1) lda + M) bytes
    M, N, K = 64, 64, 64
    fa = 2 * ((K - 1) * M + M)
    assert splan(M, N, K, (1, M), (N, 1), (N, 1), c=PA + fa)[0] == g.OK
    assert splan(M, N, K, (1, M), (N, 1), (N, 1), c=PA + fa - 2)[0] == g.ERR_OVERLAP


def test_too_large_c_leading_dimension():
    # 64 rows of C (the 64 x 64 tile) at ldc = 2^25 reach 2^31 elements: beyond the store
    # offsets
    t64 = {"tile": g.TILE_64x64x32}
    args = (256, 8, 8, 1 << 40, 2 << 40, 3 << 40, 8, 8, 1 << 25)
    assert g.gemm_f16f32_plan(*args, opts=t64)[0] == g.ERR_TOO_LARGE
    args = (256, 8, 8, 1 << 40, 2 << 40, 3 << 40, 8, 8, 1 << 24)
    assert g.gemm_f16f32_plan(*args, opts=t64)[0] == g.OK
    assert g.gemm_f16f32_plan(*args, opts={"tile": g.TILE_256x256x64})[0] == g.ERR_TOO_LARGE
    # a transposed operand's panel spans 64 k rows: 64 x lda
    assert splan(8, 8, 8, (1, 1 << 25), (8, 1), (8, 1), a=1 << 40, b=2 << 40,
                 c=3 << 40)[0] == g.ERR_TOO_LARGE
    # ... and 128 with a 128-deep tile: at ld = 2^24 + 8 that is past 2^31 for B row-major
    # (x-major), within it for the 64-deep tiles and the generic path (64 rows)
    ld = (1 << 24) + 8
    args = (8, 8, 8, 1 << 40, 2 << 40, 3 << 40, 8, ld, 8)
    assert g.gemm_f16f32_plan(*args, opts={"tile": g.TILE_32x64x128})[0] == g.ERR_TOO_LARGE
    assert g.gemm_f16f32_plan(*args, opts={"tile": g.TILE_32x64x64})[0] == g.OK
    assert g.gemm_f16f32_plan(*args, opts={"tile": g.TILE_32x64x128,
                                           "force_generic": 1})[0] == g.OK
    # a tile the planner chose itself gives way to 32 x 32 x 64 instead: 32 x 32 x 4096 takes
    # the 128-deep 32 x 64 tile from the table, and 32 x 32 x 64 at this ldb
    rc, info = g.gemm_f16f32_plan(32, 32, 4096, 1 << 40, 2 << 40, 3 << 40, 4096, 32, 32)
    assert rc == g.OK and info["tile"] == g.TILE_32x64x128
    rc, info = g.gemm_f16f32_plan(32, 32, 4096, 1 << 40, 2 << 40, 3 << 40, 4096, ld, 32)
    assert rc == g.OK and info["tile"] == g.TILE_32x32x64 and info["bk"] == 64
    # beyond what any tile addresses, still refused
    assert g.gemm_f16f32_plan(32, 32, 4096, 1 << 40, 2 << 40, 3 << 40, 4096, 1 << 25,
                              32)[0] == g.ERR_TOO_LARGE


def test_persistent_plans():
    # one round of workgroups: 256 CUs x per-CU LDS fit, a multiple of 8, at most P
    p = plan(8192, 8192, 8192, tile=g.TILE_256x256x64, persistent=g.PERSISTENT_ON)
    assert p["persistent"] == 1 and p["grid"] == 256 and p["num_programs"] == 1024
    p = plan(8192, 8192, 8192, tile=g.TILE_64x64x64, persistent=g.PERSISTENT_ON)
    assert p["grid"] == 256 * 2 and p["num_programs"] == 128 * 128     # 64 KiB of LDS each
    p = plan(512, 512, 512, tile=g.TILE_256x256x64, persistent=g.PERSISTENT_ON)
    assert p["grid"] == p["num_programs"] == 4
    p = plan(8192, 8192, 8192, tile=g.TILE_256x256x64)
    assert p["persistent"] == 0 and p["grid"] == p["num_programs"]
    # the generic path has no persistent form
    p = plan(8192, 8192, 8192, persistent=g.PERSISTENT_ON, force_generic=1)
    assert p["persistent"] == 0 and p["grid"] == p["num_programs"]
    assert g.gemm_f16f32_plan(8, 8, 8, PA, PB, PC, 8, 8, 8, opts={"persistent": 3})[0] == \
        g.ERR_OPTS


def test_misaligned_rows_keep_the_table_tile_unless_a_sliver_fits_the_ping_pong_strip():
    """Misaligned rows (odd leading dimension or a 2-byte aligned start) keep the table's
    4-wavefront 256 x 256 tile; only a right sliver of 1..16 columns moves such a problem to the
    ping-pong tile, which computes the sliver inside its own launch."""
    M = N = K = 4096
    p = plan(M, N, K)
    if p["tile"] != g.TILE_256x256x64:
        pytest.skip("the table does not pick the 4-wavefront 256 x 256 tile here")
    for kw in ({"lda": K + 1}, {"ldb": N + 1}, {"a": PA + 2}, {"lda": K + 8}):
        assert plan(M, N, K, **kw)["tile"] == g.TILE_256x256x64, kw
    p = plan(4095, 4097, 4093)
    assert p["tile"] == g.TILE_256x256x32_PP and p["strip_n"] == 1 and p["launches"] == 1
    # a wider sliver (17 columns) is split off instead, with the table's tile
    p = plan(4095, 4096 + 17, 4093)
    assert p["tile"] == g.TILE_256x256x64 and p["strip_n"] == 0 and p["launches"] == 2
    # the option to force a tile, or to keep the edges, leaves the choice alone
    assert plan(4095, 4097, 4093, split_edges=g.SPLIT_OFF)["tile"] == g.TILE_256x256x64


def test_struct_layouts_match_the_header(tmp_path):
    """Every field of gemm_f16f32_opts and gemm_f16f32_plan_info sits at the same offset (and
    each struct has the same size) in the C header, compiled by gcc, as in the ctypes binding."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "gemm_f16f32.h"',
             'int main(void) {']
    for cname, py in (("gemm_f16f32_opts", g.Opts), ("gemm_f16f32_plan_info", g.PlanInfo)):
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for field, _ in py._fields_:
            lines.append(f'  printf("{cname} {field} %zu\\n", offsetof({cname}, {field}));')
    lines += ['  return 0;', '}']
    src = tmp_path / "layout.c"
    src.write_text("\n".join(lines) + "\n")
    exe = tmp_path / "layout"
    subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"),
                    str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    got = {tuple(ln.split()[:2]): int(ln.split()[2]) for ln in out if ln}
    for cname, py in (("gemm_f16f32_opts", g.Opts), ("gemm_f16f32_plan_info", g.PlanInfo)):
        assert got[(cname, "size")] == ctypes.sizeof(py), cname
        for field, _ in py._fields_:
            assert got[(cname, field)] == getattr(py, field).offset, (cname, field)


def test_matmul_refuses_other_dtypes_before_any_gpu_call():
    torch = pytest.importorskip("torch")
    f16 = torch.zeros((4, 4), dtype=torch.float16)
    for dt in (torch.bfloat16, torch.float32, torch.int8):
        bad = torch.zeros((4, 4), dtype=dt)
        for args in ((bad, f16, f16), (f16, bad, f16), (f16, f16, bad)):
            with pytest.raises(ValueError, match="float16"):
                g.matmul(*args)
    with pytest.raises(ValueError, match="CUDA"):   # right dtype, host memory
        g.matmul(f16, f16, f16)


def test_matmul_refuses_blocks_outside_the_tensors_before_any_gpu_call():
    """The library sees pointers and strides only; the binding checks that the M x K, K x N
    and M x N blocks lie inside a, b and out (host tensors here: the check comes first)."""
    torch = pytest.importorskip("torch")
    z = lambda r, c: torch.zeros((r, c), dtype=torch.float16)
    bad = [((z(4, 8), z(7, 5), z(4, 5)), {}),                 # b has fewer rows than K
           ((z(4, 8), z(8, 5), z(3, 5)), {}),                 # out has fewer rows than M
           ((z(4, 8), z(8, 5), z(4, 4)), {}),                 # out has fewer columns than N
           ((z(4, 8), z(8, 5), z(4, 5)), dict(M=5)),
           ((z(4, 8), z(8, 5), z(4, 5)), dict(K=9)),
           ((z(4, 8), z(8, 5), z(4, 5)), dict(N=6)),
           ((z(4, 8), z(8, 5).t(), z(4, 5)), {})]             # b.t() is 5 x 8
    for args, sizes in bad:
        with pytest.raises(ValueError, match="block"):
            g.matmul(*args, **sizes)
    # blocks inside larger tensors, and empty ones, pass on to the device check
    for args, sizes in [((z(4, 8), z(9, 5), z(6, 7)), {}),
                        ((z(4, 8), z(8, 5), z(4, 5)), dict(M=2, N=3, K=1)),
                        ((z(0, 8), z(8, 5), z(0, 5)), {}),
                        ((z(4, 0), z(0, 5), z(4, 5)), {})]:
        with pytest.raises(ValueError, match="CUDA"):
            g.matmul(*args, **sizes)
    with pytest.raises(ValueError, match="CUDA"):      # out allocated for M x N
        g.matmul(z(4, 8), z(8, 5))
