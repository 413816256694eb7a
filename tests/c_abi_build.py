"""Builds tests/c_abi_check (from c_abi_check.c): plain C99 against include/gemm_f16f32.h,
linked to the in-tree libgemm_f16f32.so and the HIP runtime, found through an rpath relative
to the binary.  Called by __graft_entry__.build() after the library is built."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "c_abi_check.c")
EXE = os.path.join(HERE, "c_abi_check")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build() -> str:
    cmd = ["gcc", "-std=c99", "-Wall", "-Wextra", "-Werror", "-O2", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-L", os.path.join(ROOT, "dense_gemm_f16f32_amd"), "-lgemm_f16f32",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/../dense_gemm_f16f32_amd", "-Wl,-rpath," + os.path.join(ROCM, "lib"),
           "-o", EXE + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("gcc failed:\n" + r.stdout + r.stderr)
    os.replace(EXE + ".tmp", EXE)
    return EXE


if __name__ == "__main__":
    print(build())
