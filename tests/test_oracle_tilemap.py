"""Pins for the oracle's grouped program-id -> tile map and the XCD pre-permutation.

Source: kernl notebook "Computing coordinates on Triton GEMM example" (introduction excerpt
and cells In[1]-In[8]).  Pins: every value the notebook prints for its worked example, the
pointer printout of cell In[8] (differences only), bijection over the grid by enumeration,
the row-major (G = 1) and column-major (G >= num_pid_m) special cases, a constructive
enumeration of "groups of G tile-rows, column-major inside a group", and the partial last
group taken as printed (`pid % group_size_m`).
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_worked_example_printed_values():
    g = load("kernl_worked_example.json")
    i, p = g["inputs"], g["printed"]
    num_pid_m = oracle.cdiv(i["M"], i["BLOCK_SIZE_M"])
    num_pid_n = oracle.cdiv(i["N"], i["BLOCK_SIZE_N"])
    assert num_pid_m == p["num_pid_m"]
    assert num_pid_n == p["num_pid_n"]
    assert num_pid_n * i["GROUP_SIZE_M"] == p["num_pid_n * GROUP_SIZE_M"]
    assert num_pid_m * num_pid_n == p["nb programs to launch"]
    d = oracle.tile_map_detail(num_pid_m, num_pid_n, i["GROUP_SIZE_M"], i["pid"])
    for key in ("num_pid_in_group", "group_id", "first_pid_m", "group_size_m", "pid_m",
                "pid_n"):
        assert d[key] == p[key], key


def test_pointer_printout_differences():
    g = load("kernl_pointer_printout.json")
    pm, pn = g["pid_m"], g["pid_n"]
    BM, BN = g["BLOCK_SIZE_M"], g["BLOCK_SIZE_N"]
    lda, ldb = g["stride_am"], g["stride_bk"]

    def idx(key):
        r, c = key.strip("[]").split("][")
        return int(r), int(c)

    a0 = g["a_ptrs"]["[0][0]"]
    for key, val in g["a_ptrs"].items():
        r, k = idx(key)
        assert oracle.offset_a(pm, BM, lda, r, k) - oracle.offset_a(pm, BM, lda, 0, 0) == val - a0
    b0 = g["b_ptrs"]["[0][0]"]
    for key, val in g["b_ptrs"].items():
        k, c = idx(key)
        assert oracle.offset_b(pn, BN, ldb, k, c) - oracle.offset_b(pn, BN, ldb, 0, 0) == val - b0
    # the first element of the panel sits pid_m*BM rows / pid_n*BN columns past the base
    assert oracle.offset_a(pm, BM, lda, 0, 0) == pm * BM * lda
    assert oracle.offset_b(pn, BN, ldb, 0, 0) == pn * BN


def test_bijection_by_enumeration():
    """Every pid in [0, P) gets a distinct tile, for all num_pid_m, num_pid_n <= 40 and
    GROUP_SIZE_M <= 41 (G past num_pid_m included)."""
    for m in range(1, 41):
        for n in range(1, 41):
            for G in range(1, 42):
                t = oracle.tile_map_all(m, n, G)
                assert t[:, 0].min() >= 0 and t[:, 0].max() < m
                assert t[:, 1].min() >= 0 and t[:, 1].max() < n
                code = t[:, 0] * n + t[:, 1]
                assert np.bincount(code, minlength=m * n).max() == 1, (m, n, G)


@pytest.mark.parametrize("m,n", [(1, 1), (3, 7), (8, 12), (16, 17), (13, 5)])
def test_special_cases_row_and_column_major(m, n):
    P = m * n
    pid = np.arange(P)
    rm = oracle.tile_map_all(m, n, 1)
    assert np.array_equal(rm[:, 0], pid // n) and np.array_equal(rm[:, 1], pid % n)
    for G in (m, m + 3):
        cm = oracle.tile_map_all(m, n, G)
        assert np.array_equal(cm[:, 0], pid % m) and np.array_equal(cm[:, 1], pid // m)


@pytest.mark.parametrize("m,n,G", [(8, 12, 2), (16, 16, 4), (16, 17, 6), (32, 32, 8),
                                   (5, 3, 3), (7, 4, 3), (9, 9, 4)])
def test_constructive_grouped_order(m, n, G):
    """Groups of G tile-rows; inside a group, column after column; each column walks the
    group's rows.  In a smaller last group the printed formula starts each column at
    row first + (pid % size), a rotation of the local order; check that reading."""
    t = oracle.tile_map_all(m, n, G)
    pid = 0
    for first in range(0, m, G):
        size = min(G, m - first)
        for col in range(n):
            for r in range(size):
                if size == G or (G * n) % size == 0:
                    want_row = first + r
                else:
                    want_row = first + (pid % size)
                assert tuple(t[pid]) == (want_row, col), (pid, first, size)
                pid += 1
    assert pid == m * n


def test_partial_group_example_as_printed():
    t = oracle.tile_map_all(5, 3, 3)
    assert [tuple(x) for x in t[9:15]] == [(4, 0), (3, 0), (4, 1), (3, 1), (4, 2), (3, 2)]


def test_ragged_shape_partial_group():
    """The ragged 4095 x 4097 shape with 256 x 256 tiles and G = 6 ends in a group of 4."""
    m, n = oracle.cdiv(4095, 256), oracle.cdiv(4097, 256)
    assert (m, n) == (16, 17)
    d = oracle.tile_map_detail(m, n, 6, m * n - 1)
    assert d["first_pid_m"] == 12 and d["group_size_m"] == 4


def test_out_of_range_rejected():
    with pytest.raises(ValueError):
        oracle.tile_map(8, 12, 2, 96)
    with pytest.raises(ValueError):
        oracle.tile_map(8, 12, 0, 5)


@pytest.mark.parametrize("X", [1, 2, 8])
def test_xcd_remap_bijection_and_blocks(X):
    for P in range(1, 301):
        h = np.arange(P)
        pid = np.array([oracle.xcd_remap(P, X, int(x)) for x in h])
        assert np.array_equal(np.sort(pid), h), (P, X)
        # the workgroups dealt to one die get one contiguous run of logical ids, in order
        for x in range(X):
            mine = pid[h % X == x]
            if mine.size:
                assert np.array_equal(mine, np.arange(mine[0], mine[0] + mine.size))
        # die x owns ids [x*q + min(x, r), ...): sizes q+1 for the first r dies
        q, r = divmod(P, X)
        sizes = [int((h % X == x).sum()) for x in range(X)]
        assert sizes == [q + (1 if x < r else 0) for x in range(X)]


def test_program_tiles_composition_is_bijection():
    for (m, n, G) in [(16, 16, 4), (32, 32, 8), (16, 17, 6), (8, 12, 2)]:
        for remap in (False, True):
            t = oracle.program_tiles(m, n, G, remap)
            assert np.unique(t[:, 0]).size == m * n
            assert np.unique(t[:, 1] * n + t[:, 2]).size == m * n


def test_program_tiles_composition_hand_derived():
    """The XCD permutation is applied to the hardware id first and the grouped map to its
    result.  Worked by hand from the two definitions:
      * 8 x 12 tiles, G = 2, remap on: P = 96 = 8 x 12, so each die owns 12 consecutive
        logical ids; hardware id 1 is die 1's first workgroup -> logical id 12 -> group 0
        (24 ids), column-major over its 2 rows -> row 12 mod 2 = 0, column 12 // 2 = 6.
        Applying the map first would give the tile of id 1, (1, 0), instead.
      * 32 x 32 tiles, G = 8, remap on: die 0 receives hardware ids 0, 8, 16, ... and they
        become logical ids 0, 1, 2, ...; the first 32 of them fill rows 0-7 of columns 0-3
        (an 8 x 4 block of tiles), id t at (t mod 8, t // 8).
      * remap off: logical id = hardware id."""
    t = oracle.program_tiles(8, 12, 2, True)
    assert tuple(t[1]) == (12, 0, 6)
    assert tuple(t[0]) == (0, 0, 0)
    assert tuple(t[8]) == (1, 1, 0)          # die 0's second workgroup: logical id 1
    assert tuple(t[95]) == (95, 7, 11)       # die 7's last: 7*12 + 11 = 95
    t = oracle.program_tiles(32, 32, 8, True)
    for j in range(32):
        assert tuple(t[8 * j]) == (j, j % 8, j // 8), j
    die0 = {(int(r), int(c)) for r, c in t[0:256:8, 1:]}
    assert die0 == {(r, c) for r in range(8) for c in range(4)}
    t = oracle.program_tiles(8, 12, 2, False)
    assert tuple(t[1]) == (1, 1, 0) and tuple(t[60]) == (60, 4, 6)
