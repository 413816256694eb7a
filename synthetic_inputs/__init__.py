"""Seeded synthetic operands for the fp16 GEMM, shared by the oracle side and the HIP side.

This module only draws random operands.  It holds none of the GEMM's arithmetic: no
products, no sums, no fp32/fp64 -> fp16 narrowing of results.  Both the oracle tests
and the GPU tests/benchmark take their A and B from here, so the two sides see the same
bytes without sharing any code of the method.

Generator: SplitMix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
generators", OOPSLA 2014).  It is counter based: draw t (t = 0, 1, 2, ...) of the stream
with seed s is mix64(s + (t + 1) * 0x9E3779B97F4A7C15), where mix64 is the published
finaliser (xor-shift 30, multiply 0xBF58476D1CE4E5B9, xor-shift 27, multiply
0x94D049BB133111EB, xor-shift 31).  One stream fills A (M*K values, row-major), then B
(K*N values, row-major) continues from the next value index.

Distributions (each value is an IEEE binary16 bit pattern, returned as uint16):
  * "u(-0.5,0.5)": j = top 11 bits of the draw, value (j - 1024) / 2048.  Every value is an
    exact fp16, on a 2^-11 grid in [-0.5, 0.5).  It stands in for the matmul tutorial's
    torch.rand(fp16) - 0.5 operands (phobos "03: Matrix multiplication", check function).
  * "u(0,1)": value j / 2048, exact fp16 on a 2^-11 grid in [0, 1).  It stands in for the
    torch.rand operands of the kernl notebook's worked example ("Computing coordinates on
    Triton GEMM example", cell In[1]).
  * "n(0,0.1)": Box-Muller in float64 on the pair of draws (2*floor(t/2), 2*floor(t/2)+1),
    cos branch for even t, sin branch for odd t, times 0.1, then numpy's float64 -> float16
    conversion (round to nearest even).  Uniforms for Box-Muller are ((z >> 11) + 0.5) / 2^53.

Two low-switching-activity distributions, for measuring how much of the GEMM's time is set by
the data-dependent power of the matrix cores (same shapes, same memory traffic):
  * "zeros": every value +0 (no draw is made).
  * "s(1/64)": +1/64 or -1/64, the sign taken from the top bit of the draw: one bit of each
    operand changes from value to value.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)

DISTS = ("u(-0.5,0.5)", "u(0,1)", "n(0,0.1)")
LOW_ACTIVITY_DISTS = ("zeros", "s(1/64)")

# Draws are produced in chunks so that 8192x8192 operands do not need a 1 GiB temporary.
_CHUNK = 1 << 22


def splitmix64(seed: int, start: int, count: int) -> np.ndarray:
    """Draws start .. start+count-1 of the SplitMix64 stream with this seed (uint64)."""
    t = np.arange(start + 1, start + count + 1, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = np.uint64(seed) + t * GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


_GRID = {}


def _grid_table(dist: str) -> np.ndarray:
    """fp16 bit patterns of the 2048 grid values, indexed by the top 11 bits of a draw."""
    if dist not in _GRID:
        j = np.arange(2048, dtype=np.float64)
        v = (j - 1024.0) / 2048.0 if dist == "u(-0.5,0.5)" else j / 2048.0
        _GRID[dist] = v.astype(np.float16).view(np.uint16)
    return _GRID[dist]


def _values(dist: str, seed: int, start: int, count: int) -> np.ndarray:
    """fp16 bit patterns of values start .. start+count-1 of the stream."""
    if dist in ("u(-0.5,0.5)", "u(0,1)"):
        j = (splitmix64(seed, start, count) >> np.uint64(53)).astype(np.intp)
        return _grid_table(dist)[j]
    if dist == "n(0,0.1)":
        t = np.arange(start, start + count, dtype=np.int64)
        pair0 = (t // 2) * 2
        lo = int(pair0[0]) if count else 0
        hi = int(pair0[-1]) + 2 if count else 0
        z = splitmix64(seed, lo, hi - lo)
        u = ((z >> np.uint64(11)).astype(np.float64) + 0.5) / float(1 << 53)
        u1 = u[pair0 - lo]
        u2 = u[pair0 - lo + 1]
        r = np.sqrt(-2.0 * np.log(u1))
        ang = 2.0 * np.pi * u2
        v = np.where(t % 2 == 0, r * np.cos(ang), r * np.sin(ang)) * 0.1
        return v.astype(np.float16).view(np.uint16)
    if dist == "zeros":
        return np.zeros(count, dtype=np.uint16)
    if dist == "s(1/64)":
        sign = (splitmix64(seed, start, count) >> np.uint64(63)).astype(np.uint16)
        return np.uint16(0x2400) | (sign << np.uint16(15))   # 0x2400 = 1/64 in binary16
    raise ValueError(f"unknown distribution {dist!r}; expected one of "
                     f"{DISTS + LOW_ACTIVITY_DISTS}")


def stream(dist: str, seed: int, start: int, count: int) -> np.ndarray:
    """Values start .. start+count-1 of the seeded stream, as uint16 fp16 bit patterns.

    Chunks are independent (the generator is counter based), so they are filled by a
    small thread pool; numpy releases the GIL inside its element-wise loops.
    """
    out = np.empty(count, dtype=np.uint16)

    def fill(a: int) -> None:
        n = min(_CHUNK, count - a)
        out[a:a + n] = _values(dist, seed, start + a, n)

    starts = range(0, count, _CHUNK)
    if count <= _CHUNK:
        for a in starts:
            fill(a)
        return out
    workers = max(1, min(8, os.cpu_count() or 1))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        list(pool.map(fill, starts))
    return out


def operands(M: int, N: int, K: int, dist: str, seed: int):
    """(A, B): A is M x K and B is K x N, both row-major uint16 fp16 bit patterns.

    A takes values 0 .. M*K-1 of the stream and B the next K*N values.
    """
    A = stream(dist, seed, 0, M * K).reshape(M, K)
    B = stream(dist, seed, M * K, K * N).reshape(K, N)
    return A, B


# The five workloads: (name, M, N, K, distribution, seed).  Sizes and value ranges follow
# the matmul tutorial's 512^3 check and the notebook's 1024x768x128 worked example; the
# larger square and ragged shapes exercise the compute-bound regime and the edge masks.
WORKLOADS = (
    ("gemm512_u", 512, 512, 512, "u(-0.5,0.5)", 0),
    ("gemm1024x768x128_u01", 1024, 768, 128, "u(0,1)", 1),
    ("gemm4096_u", 4096, 4096, 4096, "u(-0.5,0.5)", 2),
    ("gemm8192_u", 8192, 8192, 8192, "u(-0.5,0.5)", 3),
    ("gemm4095x4097x4093_n", 4095, 4097, 4093, "n(0,0.1)", 4),
)


def workload(name: str):
    for w in WORKLOADS:
        if w[0] == name:
            return w
    raise KeyError(name)
