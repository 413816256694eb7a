"""The build's check of the wait states around the inline-asm 16x16x32 MFMAs (CPU only).

The 256 x 256 x 64 tile issues its MFMAs as inline asm, which the compiler's hazard checks do
not see; the code waits 32 states after the last MFMA before the accumulators are read and 8
after zeroing them before the first MFMA.  dense_gemm_f16f32_amd/build.py scans the built
gfx950 code for any accumulator move the compiler might place between them.  Checked here: the
scan flags both kinds of violation in a hand-written listing, accepts the pattern the kernels
use, and passes on the built library and on the matrix-core rate probe built beside it.
"""
import os

import pytest

from dense_gemm_f16f32_amd import build as b

KERNEL = "_ZN2gk8gemm_dmaILi256ELi256ELi64ELi2ELi1ELi2ELi2ELb1ELb0EEEvNS_4ArgsE"


def listing(*body):
    return f"0000000000001000 <{KERNEL}>:\n" + "\n".join("\t" + x for x in body) + "\n"


GOOD = listing("v_accvgpr_write_b32 a0, 0", "v_accvgpr_mov_b32 a1, a0", "s_nop 7",
               "v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]",
               "v_mfma_f32_16x16x32_f16 a[4:7], v[2:5], v[6:9], a[4:7]",
               "s_nop 7", "s_nop 7", "s_nop 7", "s_nop 7", "v_accvgpr_read_b32 v0, a0")


def test_scan_accepts_the_kernels_pattern():
    assert b.scan_mfma_waits(GOOD) == (1, [])


def test_scan_flags_a_read_before_the_drain():
    bad = listing("s_nop 7", "v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]",
                  "s_nop 7", "v_accvgpr_read_b32 v0, a3")
    n, found = b.scan_mfma_waits(bad)
    assert n == 1 and len(found) == 1 and "before the drain" in found[0]


def test_scan_flags_an_mfma_right_after_a_write():
    bad = listing("v_mfma_f32_16x16x32_f16 a[0:3], v[2:5], v[6:9], a[0:3]",
                  "s_nop 7", "s_nop 7", "s_nop 7", "s_nop 7",
                  "v_accvgpr_write_b32 a16, v92",
                  "v_mfma_f32_16x16x32_f16 a[16:19], v[4:7], v[44:47], a[16:19]")
    n, found = b.scan_mfma_waits(bad)
    assert n == 1 and len(found) == 1 and "after an accumulator write" in found[0]


def test_scan_ignores_kernels_with_compiler_managed_mfmas():
    other = GOOD.replace(KERNEL, "_ZN2gk7gemm_ppILb1ELb0ELb0EEEvNS_4ArgsE").replace(
        "s_nop 7\n\tv_mfma", "v_mfma")
    assert b.scan_mfma_waits(other) == (0, [])


def test_built_library_meets_the_waits():
    if not os.path.exists(b.SO):
        pytest.skip("library not built")
    assert b.check_mfma_waits(b.SO) >= 8


def test_built_rate_probe_meets_the_waits_and_exports_its_launcher():
    """The matrix-core rate probe (bench.py --mfma-ceiling) is built beside the library, with
    the same wait states around the asm MFMAs of both its kernels."""
    if not os.path.exists(b.PROBE_SO):
        pytest.skip("probe not built")
    assert b.check_mfma_waits(b.PROBE_SO) == 2
    import ctypes
    assert hasattr(ctypes.CDLL(b.PROBE_SO), "mfma_ceiling_launch")
