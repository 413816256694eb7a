"""Python access to the CPU oracle (oracle.c): plain fp64-sum GEMM, fp16 codec, tile map.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's CPU-baseline
leg are the only users.  Nothing in the GPU library imports, links or calls this package,
and this package imports nothing from the GPU library.

`build()` compiles oracle.c with gcc; `lib()` loads the result.  Every function here only
marshals arguments into the C library, which holds all of the oracle's arithmetic.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")

_lib = None


def build() -> str:
    """Compile oracle.c into liboracle.so (always recompiles).  Returns the path."""
    tmp = _SO + ".tmp"
    cmd = ["gcc", "-O3", "-std=c11", "-fopenmp", "-ffp-contract=off", "-Wall", "-Wextra",
           "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def lib() -> ctypes.CDLL:
    """Load liboracle.so, building it first if it is not there."""
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build()
        L = ctypes.CDLL(_SO)
        i64, u16p, i64p = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
        L.oracle_init.restype = None
        L.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_f16_to_f64.restype = ctypes.c_double
        L.oracle_f64_to_f16.argtypes = [ctypes.c_double]
        L.oracle_f64_to_f16.restype = ctypes.c_uint16
        L.oracle_gemm.argtypes = [i64, i64, i64, u16p, i64, u16p, i64, u16p, i64]
        L.oracle_gemm.restype = None
        L.oracle_gemm_plain.argtypes = [i64, i64, i64, u16p, i64, u16p, i64, u16p, i64]
        L.oracle_gemm_plain.restype = None
        L.oracle_gemm_sampled.argtypes = [i64, u16p, i64, u16p, i64, i64, i64p, i64p, u16p,
                                          ctypes.c_void_p]
        L.oracle_gemm_sampled.restype = None
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_cdiv.argtypes = [i64, i64]
        L.oracle_cdiv.restype = i64
        L.oracle_tile_map.argtypes = [i64, i64, i64, i64, ctypes.POINTER(i64),
                                      ctypes.POINTER(i64)]
        L.oracle_tile_map.restype = ctypes.c_int
        L.oracle_tile_map_detail.argtypes = [i64, i64, i64, i64, ctypes.c_void_p]
        L.oracle_tile_map_detail.restype = ctypes.c_int
        L.oracle_tile_map_fill.argtypes = [i64, i64, i64, ctypes.c_void_p, ctypes.c_void_p]
        L.oracle_tile_map_fill.restype = ctypes.c_int
        L.oracle_offset_a.argtypes = [i64, i64, i64, i64, i64]
        L.oracle_offset_a.restype = i64
        L.oracle_offset_b.argtypes = [i64, i64, i64, i64, i64]
        L.oracle_offset_b.restype = i64
        L.oracle_xcd_remap.argtypes = [i64, i64, i64]
        L.oracle_xcd_remap.restype = i64
        L.oracle_init()
        _lib = L
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _ld(a: np.ndarray) -> int:
    """Leading dimension (elements) of a row-major 2-D array with unit inner stride."""
    if a.size == 0:
        return max(a.shape[1], 1)
    assert a.strides[1] == a.itemsize and a.strides[0] % a.itemsize == 0
    return a.strides[0] // a.itemsize


def f16_to_f64(h: int) -> float:
    return lib().oracle_f16_to_f64(h)


def f64_to_f16(x: float) -> int:
    return lib().oracle_f64_to_f16(x)


def f16_decode_all() -> np.ndarray:
    """Decoded value of every one of the 65536 bit patterns, in pattern order."""
    L = lib()
    return np.array([L.oracle_f16_to_f64(h) for h in range(65536)], dtype=np.float64)


def gemm(A: np.ndarray, B: np.ndarray, C: np.ndarray | None = None, M=None, N=None, K=None,
         plain: bool = False):
    """C = fp16(sum_k A[i,k] B[k,j]) for 2-D uint16 arrays (row-major, unit inner stride).

    M, N, K default to the array shapes; A and B may be wider (their leading dimensions are
    taken from their strides).  If C is given, only its top-left M x N block is written.
    plain=True runs the one-dot-per-element form instead of the blocked one (same values:
    both add each element's products in ascending k).
    """
    assert A.dtype == np.uint16 and B.dtype == np.uint16
    M = A.shape[0] if M is None else M
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    assert A.shape[0] >= M and A.shape[1] >= K and B.shape[0] >= K and B.shape[1] >= N
    if C is None:
        C = np.zeros((M, N), dtype=np.uint16)
    assert C.dtype == np.uint16 and C.shape[0] >= M and C.shape[1] >= N
    fn = lib().oracle_gemm_plain if plain else lib().oracle_gemm
    fn(M, N, K, _ptr(A), _ld(A), _ptr(B), _ld(B), _ptr(C), _ld(C))
    return C


def gemm_sampled(A: np.ndarray, B: np.ndarray, rows, cols, K=None, want_f64: bool = False):
    """Oracle values at the listed (row, col) positions only; same semantics as gemm()."""
    K = A.shape[1] if K is None else K
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    assert rows.shape == cols.shape and rows.ndim == 1
    assert rows.size == 0 or (rows.min() >= 0 and rows.max() < A.shape[0])
    assert cols.size == 0 or (cols.min() >= 0 and cols.max() < B.shape[1])
    out = np.zeros(rows.size, dtype=np.uint16)
    f64 = np.zeros(rows.size, dtype=np.float64) if want_f64 else None
    lib().oracle_gemm_sampled(K, _ptr(A), _ld(A), _ptr(B), _ld(B),
                              rows.size, _ptr(rows), _ptr(cols), _ptr(out),
                              _ptr(f64) if want_f64 else None)
    return (out, f64) if want_f64 else out


def num_threads() -> int:
    return lib().oracle_num_threads()


def cdiv(x: int, y: int) -> int:
    return lib().oracle_cdiv(x, y)


def tile_map(num_pid_m: int, num_pid_n: int, group_size_m: int, pid: int):
    """(pid_m, pid_n) of program `pid` under the grouped order; raises on bad arguments."""
    pm, pn = ctypes.c_int64(), ctypes.c_int64()
    rc = lib().oracle_tile_map(num_pid_m, num_pid_n, group_size_m, pid, ctypes.byref(pm),
                               ctypes.byref(pn))
    if rc != 0:
        raise ValueError("tile_map: argument out of range")
    return pm.value, pn.value


def tile_map_detail(num_pid_m: int, num_pid_n: int, group_size_m: int, pid: int) -> dict:
    """The notebook's intermediate quantities for program `pid` (from the oracle's walk)."""
    out = np.zeros(6, dtype=np.int64)
    if lib().oracle_tile_map_detail(num_pid_m, num_pid_n, group_size_m, pid, _ptr(out)) != 0:
        raise ValueError("tile_map_detail: argument out of range")
    keys = ("num_pid_in_group", "group_id", "first_pid_m", "group_size_m", "pid_m", "pid_n")
    return {k: int(v) for k, v in zip(keys, out)}


def tile_map_all(num_pid_m: int, num_pid_n: int, group_size_m: int) -> np.ndarray:
    """(P, 2) array: row p is (pid_m, pid_n) of program p."""
    P = num_pid_m * num_pid_n
    pm = np.zeros(P, dtype=np.int64)
    pn = np.zeros(P, dtype=np.int64)
    if lib().oracle_tile_map_fill(num_pid_m, num_pid_n, group_size_m, _ptr(pm), _ptr(pn)) != 0:
        raise ValueError("tile_map_all: argument out of range")
    return np.stack([pm, pn], axis=1)


def offset_a(pid_m: int, BM: int, lda: int, r: int, k: int) -> int:
    return lib().oracle_offset_a(pid_m, BM, lda, r, k)


def offset_b(pid_n: int, BN: int, ldb: int, k: int, c: int) -> int:
    return lib().oracle_offset_b(pid_n, BN, ldb, k, c)


def xcd_remap(P: int, X: int, h: int) -> int:
    return lib().oracle_xcd_remap(P, X, h)


def program_tiles(num_pid_m: int, num_pid_n: int, group_size_m: int, remap: bool,
                  X: int = 8) -> np.ndarray:
    """(P, 3) array: for hardware workgroup id h, (logical pid, pid_m, pid_n).

    With remap the logical pid is xcd_remap(P, X, h), otherwise h itself; the tile is the
    grouped map of the logical pid.
    """
    P = num_pid_m * num_pid_n
    tiles = tile_map_all(num_pid_m, num_pid_n, group_size_m)
    L = lib()
    pid = np.array([L.oracle_xcd_remap(P, X, h) if remap else h for h in range(P)],
                   dtype=np.int64)
    return np.concatenate([pid[:, None], tiles[pid]], axis=1)
