"""Python binding of libgemm_f16f32.so (the gfx950 fp16/fp32-accumulate GEMM).

The functions named like the C-ABI (gemm_f16f32, gemm_f16f32_ex, gemm_f16f32_plan,
gemm_f16f32_strided, gemm_f16f32_strided_ws, gemm_f16f32_strided_scratch,
gemm_f16f32_strided_plan, gemm_f16f32_tile_map, gemm_f16f32_strerror, gemm_f16f32_version) only marshal arguments into the library; every step
of the computation runs in its HIP kernels.  `matmul` is the same call for torch tensors: it
passes their device pointers, element strides (row- or column-major, any leading dimension)
and torch's current HIP stream, and for split K a workspace tensor.  PyTorch is used for
device memory and streams only.

The library is loaded on first use; if it has not been built the call raises at once
(there is no fallback of any kind).
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libgemm_f16f32.so")

OK = 0
(ERR_DIM, ERR_NULL, ERR_LD, ERR_OVERLAP, ERR_OPTS, ERR_TOO_LARGE, ERR_HIP,
 ERR_WORKSPACE, ERR_SCRATCH) = range(-1, -10, -1)
SCRATCH_BYTES = 16 << 20   # the static split-K scratch of gemm_f16f32_strided_scratch
(TILE_AUTO, TILE_256x256x64, TILE_128x128x64, TILE_128x64x64, TILE_256x128x64,
 TILE_256x256x32, TILE_64x64x32, TILE_128x64x32, TILE_256x256x64_W8, TILE_64x64x64,
 TILE_32x32x64, TILE_32x64x64, TILE_64x32x64, TILE_32x64x128, TILE_64x64x128, TILE_32x32x128,
 TILE_64x32x128, TILE_256x256x32_PP) = range(18)
# tile id -> (BM, BN, BK, threads)
TILES = {TILE_256x256x64: (256, 256, 64, 256), TILE_128x128x64: (128, 128, 64, 256),
         TILE_128x64x64: (128, 64, 64, 256), TILE_256x128x64: (256, 128, 64, 256),
         TILE_256x256x32: (256, 256, 32, 256), TILE_64x64x32: (64, 64, 32, 256),
         TILE_128x64x32: (128, 64, 32, 256), TILE_256x256x64_W8: (256, 256, 64, 512),
         TILE_64x64x64: (64, 64, 64, 256), TILE_32x32x64: (32, 32, 64, 64),
         TILE_32x64x64: (32, 64, 64, 128), TILE_64x32x64: (64, 32, 64, 128),
         TILE_32x64x128: (32, 64, 128, 128), TILE_64x64x128: (64, 64, 128, 256),
         TILE_32x32x128: (32, 32, 128, 64), TILE_64x32x128: (64, 32, 128, 128),
         TILE_256x256x32_PP: (256, 256, 32, 512)}
PATH_DMA, PATH_GENERIC = 0, 1
REMAP_DEFAULT, REMAP_ON, REMAP_OFF = 0, 1, 2
SPLIT_DEFAULT, SPLIT_ON, SPLIT_OFF = 0, 1, 2
PERSISTENT_DEFAULT, PERSISTENT_ON, PERSISTENT_OFF = 0, 1, 2
SPLIT_K_AUTO = -1


class GemmError(RuntimeError):
    def __init__(self, code: int, what: str = ""):
        self.code = code
        super().__init__(f"{what}: {gemm_f16f32_strerror(code)} (code {code})")


class Opts(ctypes.Structure):
    _fields_ = [("tile", ctypes.c_int32), ("group_m", ctypes.c_int32),
                ("xcd_remap", ctypes.c_int32), ("force_generic", ctypes.c_int32),
                ("split_edges", ctypes.c_int32), ("persistent", ctypes.c_int32),
                ("split_k", ctypes.c_int32)]


class PlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("path", "tile", "bm", "bn", "bk", "group_m",
                                              "xcd_remap", "num_pid_m", "num_pid_n",
                                              "num_programs", "launches", "main_m", "main_n",
                                              "a_kmajor", "b_kmajor", "swapped", "threads",
                                              "persistent", "grid", "splits", "split_depth",
                                              "strip_n")
               ] + [("workspace_bytes", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {n: getattr(self, n) for n, _ in self._fields_}


_lib = None
_i64 = ctypes.c_int64
_vp = ctypes.c_void_p
_GEMM_ARGS = [_i64, _i64, _i64, _vp, _vp, _vp, _i64, _i64, _i64]
_STRIDED_ARGS = [_i64, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i64, _i64]


def lib() -> ctypes.CDLL:
    """The loaded library; raises if libgemm_f16f32.so has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(or python dense_gemm_f16f32_amd/build.py)")
        L = ctypes.CDLL(LIB_PATH)
        L.gemm_f16f32.argtypes = _GEMM_ARGS + [_vp]
        L.gemm_f16f32.restype = ctypes.c_int
        L.gemm_f16f32_ex.argtypes = _GEMM_ARGS + [_vp, ctypes.POINTER(Opts)]
        L.gemm_f16f32_ex.restype = ctypes.c_int
        L.gemm_f16f32_plan.argtypes = _GEMM_ARGS + [ctypes.POINTER(Opts),
                                                    ctypes.POINTER(PlanInfo)]
        L.gemm_f16f32_plan.restype = ctypes.c_int
        L.gemm_f16f32_strided.argtypes = _STRIDED_ARGS + [_vp, ctypes.POINTER(Opts)]
        L.gemm_f16f32_strided.restype = ctypes.c_int
        L.gemm_f16f32_strided_ws.argtypes = _STRIDED_ARGS + [_vp, _i64, _vp,
                                                             ctypes.POINTER(Opts)]
        L.gemm_f16f32_strided_ws.restype = ctypes.c_int
        L.gemm_f16f32_strided_scratch.argtypes = _STRIDED_ARGS + [_vp, ctypes.POINTER(Opts)]
        L.gemm_f16f32_strided_scratch.restype = ctypes.c_int
        L.gemm_f16f32_strided_plan.argtypes = _STRIDED_ARGS + [ctypes.POINTER(Opts),
                                                               ctypes.POINTER(PlanInfo)]
        L.gemm_f16f32_strided_plan.restype = ctypes.c_int
        L.gemm_f16f32_tile_map.argtypes = [ctypes.c_int32] * 4 + [_vp, _vp]
        L.gemm_f16f32_tile_map.restype = ctypes.c_int
        L.gemm_f16f32_strerror.argtypes = [ctypes.c_int]
        L.gemm_f16f32_strerror.restype = ctypes.c_char_p
        L.gemm_f16f32_version.argtypes = []
        L.gemm_f16f32_version.restype = ctypes.c_int
        _lib = L
    return _lib


def _opts(opts) -> Opts | None:
    if opts is None or isinstance(opts, Opts):
        return opts
    return Opts(**opts)


# ---- C-ABI names: plain integers for pointers and the stream handle -----------------------

def gemm_f16f32(M, N, K, A, B, C, lda, ldb, ldc, stream=None) -> int:
    return lib().gemm_f16f32(M, N, K, A, B, C, lda, ldb, ldc, stream)


def gemm_f16f32_ex(M, N, K, A, B, C, lda, ldb, ldc, stream=None, opts=None) -> int:
    o = _opts(opts)
    return lib().gemm_f16f32_ex(M, N, K, A, B, C, lda, ldb, ldc, stream,
                                ctypes.byref(o) if o is not None else None)


def gemm_f16f32_plan(M, N, K, A, B, C, lda, ldb, ldc, opts=None):
    """(code, dict of the plan) -- host only, nothing is launched."""
    o = _opts(opts)
    info = PlanInfo()
    rc = lib().gemm_f16f32_plan(M, N, K, A, B, C, lda, ldb, ldc,
                                ctypes.byref(o) if o is not None else None, ctypes.byref(info))
    return rc, (info.as_dict() if rc == OK else None)


def gemm_f16f32_strided(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                        stride_cm, stride_cn, stream=None, opts=None) -> int:
    o = _opts(opts)
    return lib().gemm_f16f32_strided(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn,
                                     C, stride_cm, stride_cn, stream,
                                     ctypes.byref(o) if o is not None else None)


def gemm_f16f32_strided_ws(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                           stride_cm, stride_cn, workspace, workspace_bytes, stream=None,
                           opts=None) -> int:
    o = _opts(opts)
    return lib().gemm_f16f32_strided_ws(M, N, K, A, stride_am, stride_ak, B, stride_bk,
                                        stride_bn, C, stride_cm, stride_cn, workspace,
                                        workspace_bytes, stream,
                                        ctypes.byref(o) if o is not None else None)


def gemm_f16f32_strided_scratch(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                                stride_cm, stride_cn, stream=None, opts=None) -> int:
    o = _opts(opts)
    return lib().gemm_f16f32_strided_scratch(M, N, K, A, stride_am, stride_ak, B, stride_bk,
                                             stride_bn, C, stride_cm, stride_cn, stream,
                                             ctypes.byref(o) if o is not None else None)


def gemm_f16f32_strided_plan(M, N, K, A, stride_am, stride_ak, B, stride_bk, stride_bn, C,
                             stride_cm, stride_cn, opts=None):
    """(code, dict of the plan) -- host only, nothing is launched."""
    o = _opts(opts)
    info = PlanInfo()
    rc = lib().gemm_f16f32_strided_plan(M, N, K, A, stride_am, stride_ak, B, stride_bk,
                                        stride_bn, C, stride_cm, stride_cn,
                                        ctypes.byref(o) if o is not None else None,
                                        ctypes.byref(info))
    return rc, (info.as_dict() if rc == OK else None)


def gemm_f16f32_tile_map(num_pid_m, num_pid_n, group_m, xcd_remap, out_dev, stream=None) -> int:
    return lib().gemm_f16f32_tile_map(num_pid_m, num_pid_n, group_m, xcd_remap, out_dev, stream)


def gemm_f16f32_strerror(code: int) -> str:
    return lib().gemm_f16f32_strerror(code).decode()


def gemm_f16f32_version() -> int:
    return lib().gemm_f16f32_version()


# ---- torch tensors -------------------------------------------------------------------------

def _stream_handle(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def matmul(a, b, out=None, *, M=None, N=None, K=None, stream=None, workspace=None, **opts):
    """out[:M, :N] = fp16(a[:M, :K] @ b[:K, :N]) on the GPU (fp32 accumulation).

    a, b, out: 2-D CUDA tensors of float16 (or int16 / uint16 holding float16 bits; bfloat16
    and other dtypes are refused),
    each row-major or column-major (one unit stride) with any leading dimension: transposed
    views such as `w.t()` are read in place.  opts: tile, group_m, xcd_remap, force_generic,
    split_edges, persistent, split_k (see include/gemm_f16f32.h).  Split K goes through
    gemm_f16f32_strided_ws: with split_k >= 2 or SPLIT_K_AUTO, and also whenever a
    `workspace` (a CUDA tensor) is given, split_k then defaulting to SPLIT_K_AUTO.  A needed
    workspace that is not given is allocated by torch for this call.  Raises GemmError on a
    non-zero return code.  Launches on torch's current stream unless `stream` is given.
    The M x K, K x N and M x N blocks must lie inside a, b and out (ValueError otherwise):
    the library sees only pointers and strides, so it cannot check a tensor's extent.
    """
    import torch
    fp16_bits = (torch.float16, torch.int16) + ((torch.uint16,) if hasattr(torch, "uint16")
                                                  else ())
    for t in (a, b) if out is None else (a, b, out):
        if t.dim() != 2:
            raise ValueError("expected 2-D tensors")
        if t.dtype not in fp16_bits:   # bfloat16 is 2 bytes too, but not these bits
            raise ValueError(f"operands must be float16 (or int16/uint16 holding float16 "
                             f"bits), got {t.dtype}")
    M = a.shape[0] if M is None else M
    K = a.shape[1] if K is None else K
    N = b.shape[1] if N is None else N
    # Negative sizes are left to the library, which returns ERR_DIM for them.
    for t, rows, cols, what in ((a, M, K, "a"), (b, K, N, "b")) + (
            () if out is None else ((out, M, N, "out"),)):
        if rows > t.shape[0] or cols > t.shape[1]:
            raise ValueError(f"{what} is {tuple(t.shape)}; the call needs its first "
                             f"{rows} x {cols} block (M={M}, N={N}, K={K})")
    if not all(t.is_cuda for t in ((a, b) if out is None else (a, b, out))):
        raise ValueError("operands must be CUDA tensors")
    # Memory this call allocates belongs to the stream the kernels run on: torch's caching
    # allocator hands a freed block out again only to work on its own stream, so the
    # workspace freed on return cannot be reused by other streams while the kernels still use
    # it.
    s = torch.cuda.current_stream() if stream is None else stream
    if out is None:
        with torch.cuda.stream(s):
            out = torch.empty((max(M, 0), max(N, 0)), dtype=a.dtype, device=a.device)
    args = (M, N, K, a.data_ptr(), a.stride(0), a.stride(1), b.data_ptr(), b.stride(0),
            b.stride(1), out.data_ptr(), out.stride(0), out.stride(1))
    if workspace is not None and "split_k" not in opts:
        opts = dict(opts, split_k=SPLIT_K_AUTO)
    o = Opts(**opts) if opts else None
    if o is None or o.split_k in (0, 1):
        rc = gemm_f16f32_strided(*args, s.cuda_stream, o)
        if rc != OK:
            raise GemmError(rc, "gemm_f16f32_strided")
        return out
    if workspace is None:
        rc, info = gemm_f16f32_strided_plan(*args, opts=o)
        if rc != OK:
            raise GemmError(rc, "gemm_f16f32_strided_plan")
        if info["workspace_bytes"] > 0:
            with torch.cuda.stream(s):
                workspace = torch.empty(info["workspace_bytes"], dtype=torch.uint8,
                                        device=out.device)
    ptr, nbytes = (0, 0) if workspace is None else (workspace.data_ptr(),
                                                    workspace.numel() * workspace.element_size())
    rc = gemm_f16f32_strided_ws(*args, ptr, nbytes, s.cuda_stream, o)
    if rc != OK:
        raise GemmError(rc, "gemm_f16f32_strided_ws")
    return out


def tile_map(num_pid_m, num_pid_n, group_m, xcd_remap, stream=None):
    """(P, 3) int32 CUDA tensor from gemm_f16f32_tile_map: (logical pid, pid_m, pid_n)."""
    import torch
    P = num_pid_m * num_pid_n
    out = torch.full((P, 3), -1, dtype=torch.int32, device="cuda")
    rc = gemm_f16f32_tile_map(num_pid_m, num_pid_n, group_m, xcd_remap, out.data_ptr(),
                              _stream_handle(stream))
    if rc != OK:
        raise GemmError(rc, "gemm_f16f32_tile_map")
    return out
