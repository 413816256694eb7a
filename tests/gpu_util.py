"""Helpers shared by the GPU tests: device transfer of fp16 bit patterns and the tolerance.

Acceptance (per element): |gpu - oracle| <= 1e-2 + 2^-10 |oracle|.  The absolute part is the
matmul tutorial's own allclose tolerance (phobos "03: Matrix multiplication", check
function); the relative part admits the one-ulp flip an fp32 sum in a different order can
cause when it is narrowed to fp16 (one fp16 ulp is at most 2^-10 of the value).  Infinities
must match exactly and NaN must meet NaN.
"""
import numpy as np

ATOL = 1e-2
RTOL = 2.0 ** -10


def to_dev(a_u16: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a_u16).view(np.int16)).cuda()


def from_dev(t) -> np.ndarray:
    return t.cpu().numpy().view(np.uint16)


def f64(bits) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def tolerance_report(gpu_bits, oracle_bits):
    """(ok, violations, worst |err| / bound) for equal-shaped arrays of fp16 patterns."""
    g = f64(gpu_bits)
    o = f64(oracle_bits)
    nan_g, nan_o = np.isnan(g), np.isnan(o)
    inf_o = np.isinf(o)
    bad = (nan_g != nan_o)
    bad |= inf_o & ~nan_g & (g != o)
    fin = ~nan_o & ~inf_o
    err = np.where(fin, np.abs(g - o), 0.0)
    bound = ATOL + RTOL * np.abs(np.where(fin, o, 0.0))
    bad |= fin & ~(err <= bound)
    worst = float(np.max(err / bound)) if err.size else 0.0
    return (not bad.any()), int(bad.sum()), worst


def assert_within_tolerance(gpu_bits, oracle_bits, what=""):
    ok, nbad, worst = tolerance_report(gpu_bits, oracle_bits)
    assert ok, f"{what}: {nbad} elements outside 1e-2 + 2^-10|oracle| (worst ratio {worst:.3g})"
    return worst
