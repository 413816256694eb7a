"""Compile the HIP library (libgemm_f16f32.so) for gfx950, in-tree.

Every call recompiles.  Flags: -O3 for gfx950 only; packed fp32 arithmetic is disabled
(`-packed-fp32-ops`), so the compiler emits no packed-fp32 vector ops.  After compiling, the
wait states around the inline-asm MFMAs are checked in the built code (check_mfma_waits).
"""
from __future__ import annotations

import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "gemm_f16f32.hip")
SO = os.path.join(PKG, "libgemm_f16f32.so")
# The matrix-core rate probe (measurement only: bench.py --mfma-ceiling).
PROBE_SRC = os.path.join(PKG, "csrc", "mfma_ceiling.hip")
PROBE_SO = os.path.join(PKG, "libmfma_ceiling.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wall", "-Wno-unused-function"]


LLVM = os.path.join(os.environ.get("ROCM_PATH", "/opt/rocm"), "llvm", "bin")

KERNEL_SOURCES = ("gemm_kernels.hpp", "gemm_tiles.hpp")


def strip_comments(text: str) -> str:
    """C++ source without comments and with runs of white space collapsed (the sources have
    no string literals that contain comment markers)."""
    import re
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash() -> str:
    """sha256 (first 16 hex digits) of the files that fix the kernels' code -- the device code
    and the tile configurations -- with comments and white space removed, so that only a code
    change counts.  The planner and its dispatch table are left out: they choose the launch
    configuration.  The dispatch table and the HBM-traffic record carry the hash they were
    measured at."""
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(PKG, "csrc", name)) as f:
            h.update(name.encode() + b"\0" + strip_comments(f.read()).encode())
    return h.hexdigest()[:16]

# Kernels whose 16x16x32 MFMAs are inline asm (the 256 x 256 x 64 tile on 2 x 2 wavefronts:
# its DMA, persistent, split-K and generic forms).  The compiler's hazard checks do not see
# those MFMAs, so the code provides the wait states itself (gemm_kernels.hpp, mfma16).
ASM_MFMA_KERNELS = ("mfma_ceiling",                         # the rate probe (both)
                    "ILi256ELi256ELi64ELi2ELi1ELi2ELi2E",   # gemm_dma*, tile 1
                    "gemm_genericILi256ELi256ELb")          # gemm_generic, 256 x 256 tiles


def _asm_mfma_kernel(name: str) -> bool:
    return any(k in name for k in ASM_MFMA_KERNELS) and (
        "gemm_generic" not in name or "ELi2ELi2ELb" in name)


def disassemble(so_path: str) -> str:
    """AMD assembly of the gfx950 code object inside a library built here."""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        fat, co = os.path.join(d, "fatbin"), os.path.join(d, "gfx950.co")
        # an explicit output file: without one objcopy rewrites its input in place
        subprocess.run(["objcopy", "--dump-section", f".hip_fatbin={fat}", so_path,
                        os.path.join(d, "copy.so")], check=True, capture_output=True)
        subprocess.run([os.path.join(LLVM, "clang-offload-bundler"), "--unbundle", "--type=o",
                        f"--input={fat}", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--output={co}"], check=True, capture_output=True)
        return subprocess.run([os.path.join(LLVM, "llvm-objdump"), "-d", "--mcpu=gfx950", co],
                              check=True, capture_output=True, text=True).stdout


def scan_mfma_waits(asm: str):
    """Scans the asm-MFMA kernels of a disassembly, in program order: after an MFMA that
    writes accumulator registers, no v_accvgpr_read/mov may come before the drain (four
    `s_nop 7`, 32 wait states); after a v_accvgpr_write/mov, no MFMA may come before an
    `s_nop 7` (the pin's 8 wait states).  Returns (kernels checked, violations)."""
    import re
    checked, bad = 0, []
    for block in re.split(r"\n(?=[0-9a-f]+ <)", asm):
        m = re.match(r"[0-9a-f]+ <([^>]+)>:", block)
        if not m or not _asm_mfma_kernel(m.group(1)):
            continue
        checked += 1
        mfma_pending = write_pending = False
        nops = 0
        for line in block.splitlines()[1:]:
            ins = line.strip().split("//")[0].strip()
            op = ins.split(" ")[0] if ins else ""
            if op == "s_nop" and ins.endswith(" 7"):
                nops += 1
                write_pending = False
                if nops >= 4:
                    mfma_pending = False
                continue
            nops = 0
            if op.startswith("v_mfma"):
                if write_pending:
                    bad.append(f"{m.group(1)}: MFMA right after an accumulator write: {ins}")
                if ins.split(" ")[1].startswith("a["):
                    mfma_pending = True
            elif op in ("v_accvgpr_read_b32", "v_accvgpr_mov_b32") and mfma_pending:
                bad.append(f"{m.group(1)}: accumulator read before the drain: {ins}")
            if op in ("v_accvgpr_write_b32", "v_accvgpr_mov_b32"):
                write_pending = True
    return checked, bad


def check_mfma_waits(so_path: str) -> int:
    """scan_mfma_waits on a built library; raises on a violation (which would mean the compiler
    moved accumulators around the asm MFMAs) and returns the number of kernels checked."""
    checked, bad = scan_mfma_waits(disassemble(so_path))
    if bad:
        raise RuntimeError("asm MFMA wait states not met:\n" + "\n".join(bad[:20]))
    return checked


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
    n = check_mfma_waits(tmp)
    if n == 0:
        os.remove(tmp)
        raise RuntimeError("no asm-MFMA kernel found to check in the built library")
    os.replace(tmp, SO)
    build_probe()
    return SO


def build_probe() -> str:
    """Compiles the matrix-core rate probe (a library of its own, for bench.py only)."""
    tmp = PROBE_SO + ".tmp"
    r = subprocess.run([HIPCC, *FLAGS, PROBE_SRC, "-o", tmp], capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on the probe:\n" + "\n".join(msgs))
    if check_mfma_waits(tmp) != 2:
        os.remove(tmp)
        raise RuntimeError("the probe's two asm-MFMA kernels were not found to check")
    os.replace(tmp, PROBE_SO)
    return PROBE_SO


if __name__ == "__main__":
    print(build())
