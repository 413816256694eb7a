"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

* oracle/oracle.c, built with gcc and the sanitizers, driven by tests/sanitize_oracle.c through
  every function on edge inputs (exact-size heap buffers, so any read or write past one is
  reported).
* The library's host side (gemm_f16f32.hip compiled host-only: validation, storage-order
  normalisation, tile choice, edge split, split K, error strings), driven by
  tests/sanitize_host.c over a million seeded argument sets, valid and invalid.  That program
  runs without a GPU and without the HIP runtime: it defines the few runtime entry points the
  host side imports (kernel registration no-ops, a launch that fails), and it checks that no
  call it makes -- plans, and calls whose plan was refused or empty -- attempts a launch.
Any sanitizer finding aborts the program, and the test fails with its report.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLANG = os.path.join(ROCM, "llvm", "bin", "clang")
CLANGXX = os.path.join(ROCM, "llvm", "bin", "clang++")
SAN_ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=600, **kw)
    assert r.returncode == 0, " ".join(map(str, cmd)) + "\n" + r.stdout + r.stderr
    return r.stdout


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    exe = tmp_path / "san_oracle"
    run(["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "sanitize_oracle.c"),
         "-lm", "-o", str(exe)])
    assert run([str(exe)], env=SAN_ENV).strip().endswith("ok")


def test_library_host_side_under_sanitizers(tmp_path):
    if not (os.path.exists(CLANG) and os.path.exists(CLANGXX)):
        pytest.skip("ROCm clang not available")
    obj, lib = tmp_path / "gemm_san.o", tmp_path / "libgemm_san.so"
    # host-only compile: no device code is built, the sanitizers apply to the host pass only
    run([CLANGXX, "-x", "hip", "--offload-arch=gfx950", "--cuda-host-only", "-O1", "-g",
         "-std=c++17", "-fPIC",
         "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
         "-Xarch_host", "-fno-sanitize-recover=all",
         "-I", os.path.join(ROOT, "include"),
         "-I", os.path.join(ROOT, "dense_gemm_f16f32_amd", "csrc"),
         "-c", os.path.join(ROOT, "dense_gemm_f16f32_amd", "csrc", "gemm_f16f32.hip"),
         "-o", str(obj)])
    run([CLANGXX, "-shared", "-Xarch_host", "-fsanitize=address",
         "-Xarch_host", "-fsanitize=undefined", str(obj), "-o", str(lib)])
    undefined = run(["nm", "-u", str(lib)])
    fatbin = [ln.split()[-1] for ln in undefined.splitlines() if "__hip_fatbin" in ln]
    assert len(fatbin) == 1, undefined
    exe = tmp_path / "san_host"
    run([CLANG, "-std=c99", "-O1", "-g", "-fsanitize=address,undefined",
         "-fno-sanitize-recover=all", "-Wall", "-Wextra", "-Werror", f"-DFATBIN_SYM={fatbin[0]}",
         "-I", os.path.join(ROOT, "include"), os.path.join(HERE, "sanitize_host.c"),
         "-L", str(tmp_path), "-lgemm_san", f"-Wl,-rpath,{tmp_path}", "-rdynamic",
         "-o", str(exe)])
    out = run([str(exe)], env=SAN_ENV)
    assert out.strip().endswith("ok"), out
