"""Compile the HIP library (libgemm_f16f32.so) for gfx950, in-tree.

Every call recompiles.  Flags: -O3 for gfx950 only; packed fp32 arithmetic is disabled
(`-packed-fp32-ops`), so the compiler emits no packed-fp32 vector ops.
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gemm_f16f32.hip")
SO = os.path.join(PKG, "libgemm_f16f32.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


def build(extra=()) -> str:
    tmp = SO + ".tmp"
    cmd = [HIPCC, *FLAGS, *extra, "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(PKG, "csrc"), SRC, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass does not know the packed-fp32 feature and says so; that is harmless.
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if msgs:
        print("\n".join(msgs))
    # Every kernel must have its host launch stub; an undefined one means the host pass
    # dropped a kernel and the library would fail to load.
    nm = subprocess.run(["nm", "-D", "--undefined-only", tmp], capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in nm.stdout.splitlines() if "__device_stub__" in ln]
    if nm.returncode != 0 or missing:
        os.remove(tmp)
        raise RuntimeError("undefined kernel stubs in the built library: " + ", ".join(missing))
    os.replace(tmp, SO)
    return SO


if __name__ == "__main__":
    print(build())
