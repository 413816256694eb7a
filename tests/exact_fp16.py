"""Exact integer arithmetic on IEEE binary16 values, for pinning the oracle.

Independent of the oracle's code: values are handled as integers times 2^-24 (every finite
fp16 is one), products as integers times 2^-48, sums exactly, and the final rounding to
fp16 (nearest, ties to even, overflow to infinity) is done with integer division.  Only
finite inputs are handled.
"""
from __future__ import annotations

import numpy as np


def f16_to_int24(h: int) -> int:
    """The finite fp16 with bit pattern h, as the integer n with value n * 2^-24."""
    s = -1 if (h >> 15) & 1 else 1
    e = (h >> 10) & 0x1F
    f = h & 0x3FF
    if e == 31:
        raise ValueError("non-finite input")
    if e == 0:
        return s * f
    return s * ((1024 + f) << (e - 1))


def _div_round_half_even(a: int, d: int) -> int:
    """round(a / d) for a >= 0, d > 0, ties to even."""
    q, r = divmod(a, d)
    if 2 * r > d or (2 * r == d and q % 2 == 1):
        q += 1
    return q


def round_scaled_to_f16(n: int, scale: int) -> int:
    """Bit pattern of the fp16 nearest to n * 2^-scale (ties to even; overflow to inf).

    Zero gives +0 (0x0000).
    """
    if n == 0:
        return 0
    sign = 0x8000 if n < 0 else 0
    a = -n if n < 0 else n
    # unbiased exponent E with 2^E <= a * 2^-scale < 2^(E+1)
    E = a.bit_length() - 1 - scale
    if E < -14:
        # subnormal spacing 2^-24: m = round(a * 2^-scale / 2^-24)
        shift = scale - 24
        m = _div_round_half_even(a, 1 << shift) if shift >= 0 else a << -shift
        return sign | m            # m == 1024 is exactly the smallest normal's pattern
    # normal: spacing 2^(E-10); 11-bit significand q in [1024, 2048]
    shift = scale + E - 10
    q = _div_round_half_even(a, 1 << shift) if shift >= 0 else a << -shift
    if q == 2048:
        q = 1024
        E += 1
    if E > 15:
        return sign | 0x7C00
    return sign | ((E + 15) << 10) | (q - 1024)


def gemm_exact(A: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Correctly rounded fp16 result of the exact sum of products, for small finite inputs."""
    M, K = A.shape
    K2, N = B.shape
    assert K == K2
    a = [[f16_to_int24(int(A[i, k])) for k in range(K)] for i in range(M)]
    b = [[f16_to_int24(int(B[k, j])) for j in range(N)] for k in range(K)]
    C = np.zeros((M, N), dtype=np.uint16)
    for i in range(M):
        for j in range(N):
            s = 0
            for k in range(K):
                s += a[i][k] * b[k][j]
            C[i, j] = round_scaled_to_f16(s, 48)
    return C
