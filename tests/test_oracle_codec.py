"""Pins for the oracle's fp16 codec (decode exactly, encode to nearest with ties to even).

The narrowing mode is the one the matmul tutorial's `.to(float16)` implies (phobos
"03: Matrix multiplication", paragraph after the kernel): IEEE round to nearest, ties to
even.  Checks: exhaustive agreement with numpy's independent binary16 conversion, every
midpoint between neighbouring fp16 values, overflow edges, and integer exact rounding.
"""
import numpy as np
import pytest

import oracle
from exact_fp16 import f16_to_int24, round_scaled_to_f16


@pytest.fixture(scope="module")
def decoded():
    return oracle.f16_decode_all()


def test_decode_all_patterns_match_numpy(decoded):
    ref = np.arange(65536, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(decoded), nan)
    assert np.array_equal(decoded[~nan], ref[~nan])
    # sign of zero and of infinities preserved
    assert np.array_equal(np.signbit(decoded[~nan]), np.signbit(ref[~nan]))


def test_decode_matches_integer_definition(decoded):
    for h in range(65536):
        if (h >> 10) & 0x1F == 31:
            continue
        assert decoded[h] == f16_to_int24(h) * 2.0 ** -24


def test_roundtrip_every_pattern(decoded):
    L = oracle.lib()
    for h in range(65536):
        back = L.oracle_f64_to_f16(float(decoded[h]))
        if np.isnan(decoded[h]):
            assert (back & 0x7C00) == 0x7C00 and (back & 0x3FF) != 0
            assert (back >> 15) == (h >> 15)
        else:
            assert back == h, hex(h)


def test_midpoints_round_to_even(decoded):
    """Every exact midpoint between adjacent finite non-negative fp16 values."""
    L = oracle.lib()
    for h in range(0, 0x7BFF):
        lo, hi = decoded[h], decoded[h + 1]
        mid = (lo + hi) / 2.0            # exact in double
        want = h if h % 2 == 0 else h + 1
        assert L.oracle_f64_to_f16(mid) == want, hex(h)
        assert L.oracle_f64_to_f16(-mid) == (want | 0x8000), hex(h)
        # just off the midpoint goes to the nearer neighbour
        assert L.oracle_f64_to_f16(np.nextafter(mid, -np.inf)) == h
        assert L.oracle_f64_to_f16(np.nextafter(mid, np.inf)) == h + 1


def test_overflow_edges():
    L = oracle.lib()
    assert L.oracle_f64_to_f16(65504.0) == 0x7BFF
    assert L.oracle_f64_to_f16(65519.99) == 0x7BFF
    assert L.oracle_f64_to_f16(65520.0) == 0x7C00          # tie between 65504 and 2^16 -> inf
    assert L.oracle_f64_to_f16(-65520.0) == 0xFC00
    assert L.oracle_f64_to_f16(1e300) == 0x7C00
    assert L.oracle_f64_to_f16(0.0) == 0x0000
    assert L.oracle_f64_to_f16(-0.0) == 0x8000
    assert L.oracle_f64_to_f16(2.0 ** -25) == 0x0000       # tie between 0 and 2^-24 -> 0
    assert L.oracle_f64_to_f16(3 * 2.0 ** -25) == 0x0002   # tie between 1 and 2 ulps -> 2
    assert L.oracle_f64_to_f16(2.0 ** -26) == 0x0000


def test_encode_matches_numpy_on_random_doubles():
    rng = np.random.default_rng(123)
    L = oracle.lib()
    mags = np.exp(rng.uniform(np.log(2.0 ** -30), np.log(70000.0), 20000))
    xs = mags * rng.choice([-1.0, 1.0], mags.size)
    with np.errstate(over="ignore"):
        want = xs.astype(np.float16).view(np.uint16)
    got = np.array([L.oracle_f64_to_f16(float(x)) for x in xs], dtype=np.uint16)
    assert np.array_equal(got, want)


def test_encode_matches_integer_rounding():
    """Random integers times 2^-48 (the grid of fp16 product sums) rounded exactly."""
    rng = np.random.default_rng(7)
    L = oracle.lib()
    for _ in range(20000):
        n = int(rng.integers(-(1 << 62), 1 << 62)) >> int(rng.integers(0, 62))
        x = n * 2.0 ** -48
        if float(n) != n:        # keep cases whose double value is exactly n * 2^-48
            continue
        assert L.oracle_f64_to_f16(x) == round_scaled_to_f16(n, 48)
