"""Helpers shared by the GPU tests: device transfer of fp16 bit patterns, the tolerance,
padded storage with canaries, sampled positions and checksums.

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


# ---- storage with padding and canaries (strided layouts) ------------------------------
NAN = 0x7E00
CANARY = 0x5A5A


def place(X, col_major, pad=0, offset=0, fill=NAN):
    """Device copy of the logical R x S matrix X (fp16 bits) stored row- or column-major with
    `pad` extra elements per stored row and its first element `offset` elements into the
    buffer.  Returns the logical (R, S) view (a transposed view when column-major)."""
    import torch
    stored = np.ascontiguousarray(X.T if col_major else X)
    rows, cols = stored.shape
    ld = cols + pad
    buf = torch.full((offset + rows * ld + 8,), fill, dtype=torch.int16, device="cuda")
    body = buf[offset:offset + rows * ld].view(rows, ld)
    body[:, :cols] = to_dev(stored)
    view = body[:, :cols]
    return view.t() if col_major else view


def output(M, N, col_major, pad=3):
    return place(np.zeros((M, N), np.uint16), col_major, pad, fill=CANARY)


def padding_untouched(C_view, col_major):
    """The ld padding of C's storage still holds the canary."""
    import torch
    stored = C_view.t() if col_major else C_view
    rows, cols = stored.shape
    ld = stored.stride(0)
    flat = torch.as_strided(stored, (rows, ld), (ld, 1))
    return bool((flat[:, cols:] == CANARY).all())


# ---- full-size workloads: sampled elements and checksums --------------------------------
def sample_positions(M, N, bm, bn, per_tile, seed):
    """Per output tile: its four corners plus `per_tile` random elements; plus C's corners."""
    rng = np.random.default_rng(seed)
    rows, cols = [], []
    for tm in range(0, M, bm):
        for tn in range(0, N, bn):
            r1, c1 = min(tm + bm, M) - 1, min(tn + bn, N) - 1
            rows += [tm, tm, r1, r1]
            cols += [tn, c1, tn, c1]
            rows += list(rng.integers(tm, r1 + 1, per_tile))
            cols += list(rng.integers(tn, c1 + 1, per_tile))
    rows += [0, 0, M - 1, M - 1]
    cols += [0, N - 1, 0, N - 1]
    return np.array(rows, dtype=np.int64), np.array(cols, dtype=np.int64)


def checksum_ok(A, B, C):
    """Row and column sums of C against A (B 1) and (1^T A) B in fp64: a coarse extra check.

    Each C element is within 1e-2 + 2^-10 |C| of the exact sum, so a row's total error is
    within N * 1e-2 + 2^-10 sum|C| (and likewise per column).  The bound is loose (about 100
    per row at N = 8192): a wrong or missing tile row or column band breaks it, but a single
    wrong element or one dropped k panel in one tile can pass, so it never replaces the
    element-wise comparison.
    """
    a, b, c = f64(A), f64(B), f64(C)
    row_want = a @ b.sum(axis=1)
    col_want = a.sum(axis=0) @ b
    row_err = np.abs(c.sum(axis=1) - row_want)
    col_err = np.abs(c.sum(axis=0) - col_want)
    row_bound = c.shape[1] * 1e-2 + 2.0 ** -10 * np.abs(c).sum(axis=1)
    col_bound = c.shape[0] * 1e-2 + 2.0 ** -10 * np.abs(c).sum(axis=0)
    return bool(np.all(row_err <= row_bound) and np.all(col_err <= col_bound))
