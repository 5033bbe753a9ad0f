"""FP16 GEMM and GEMV for AMD MI355X (gfx950) behind a small C ABI.

    gemm_f16(A, B, D=None)   D = A · Bᵀ   A [M,K], B [N,K], D [M,N]  (fp16, FP32 accumulate)
    gemv_f16(x, W, y=None)   y = x · Wᵀ   x [K],   W [N,K], y [N]

This module only marshals arguments: it checks tensor dtypes, devices and
shapes, passes raw device pointers, sizes and the current HIP stream to
libgemvtile.so (see include/gemvtile.h), and turns a nonzero status into an
exception.  Every step of the computation runs in the library's HIP kernels;
there is no fallback path.  If the library has not been built, importing
works but every call raises ``GemvTileLibraryMissing``.
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GemvTileError",
    "GemvTileLibraryMissing",
    "LIBRARY_PATH",
    "EXPORTED_SYMBOLS",
    "load_library",
    "gemm_f16",
    "gemv_f16",
    "gemm_f16_ptr",
    "gemv_f16_ptr",
    "gemm_bf16",
    "gemv_bf16",
    "gemm_bf16_ptr",
    "gemv_bf16_ptr",
    "gemm_bias_f16",
    "gemm_bias_bf16",
    "gemm_splitk_f16",
    "gemm_splitk_bf16",
    "gemm_splitk_f16_noalloc",
    "splitk_splits",
    "splitk_workspace_bytes",
    "ACT_NONE",
    "ACT_RELU",
    "gemm_f16_variant",
    "gemv_f16_variant",
    "status_string",
    "tile_coord",
    "xcd_logical_id",
    "gemm_config",
    "gemm_grid",
    "gemm_tile",
    "gemv_grid",
    "device_caps",
    "ring_trace",
    "alloc_splitk_workspace",
]

LIBRARY_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libgemvtile.so")

# Every symbol include/gemvtile.h declares.
EXPORTED_SYMBOLS = (
    "gemm_f16",
    "gemv_f16",
    "gemm_bf16",
    "gemv_bf16",
    "gemm_bias_f16",
    "gemm_bias_bf16",
    "gemm_splitk_f16",
    "gemm_splitk_bf16",
    "gemm_splitk_f16_noalloc",
    "gemvtile_gemm_splitk_splits",
    "gemvtile_gemm_splitk_workspace",
    "gemvtile_status_string",
    "gemvtile_tile_coord",
    "gemvtile_gemm_config",
    "gemvtile_gemm_grid",
    "gemvtile_gemm_tile",
    "gemvtile_gemv_grid",
    "gemvtile_device_caps",
    "gemvtile_ring_trace",
    "gemvtile_gemm_f16_variant",
    "gemvtile_gemm_f16_timed",
    "gemvtile_gemv_f16_variant",
    "gemvtile_xcd_logical_id",
)

STATUS_NAMES = {
    0: "GEMVTILE_OK",
    1: "GEMVTILE_ERR_INVALID_ARG",
    2: "GEMVTILE_ERR_UNSUPPORTED",
    3: "GEMVTILE_ERR_LAUNCH",
    4: "GEMVTILE_ERR_DEVICE",
    5: "GEMVTILE_ERR_SCRATCH",
}


class GemvTileLibraryMissing(RuntimeError):
    """libgemvtile.so is not built (run __graft_entry__.build())."""


class GemvTileError(RuntimeError):
    """A library call returned a nonzero status."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None


def load_library(path: str = LIBRARY_PATH) -> ctypes.CDLL:
    """Load libgemvtile.so (once) and declare its signatures."""
    global _lib
    if _lib is not None and path == LIBRARY_PATH:
        return _lib
    if not os.path.exists(path):
        raise GemvTileLibraryMissing(f"{path} not found; build it with __graft_entry__.build()")
    lib = ctypes.CDLL(path)
    vp, i64, c_int = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
    i64p = ctypes.POINTER(ctypes.c_int64)
    intp = ctypes.POINTER(ctypes.c_int)
    lib.gemm_f16.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.gemm_f16.restype = c_int
    lib.gemv_f16.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.gemv_f16.restype = c_int
    lib.gemm_bias_f16.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, vp]
    lib.gemm_bias_f16.restype = c_int
    lib.gemm_bias_bf16.argtypes = [vp, vp, vp, vp, i64, i64, i64, c_int, vp]
    lib.gemm_bias_bf16.restype = c_int
    lib.gemm_splitk_f16.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp]
    lib.gemm_splitk_f16.restype = c_int
    lib.gemm_splitk_bf16.argtypes = [vp, vp, vp, i64, i64, i64, vp, i64, vp]
    lib.gemm_splitk_bf16.restype = c_int
    lib.gemvtile_gemm_f16_timed.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64]
    lib.gemvtile_gemm_f16_timed.restype = c_int
    lib.gemm_splitk_f16_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.gemm_splitk_f16_noalloc.restype = c_int
    lib.gemvtile_gemm_splitk_splits.argtypes = [i64, i64, i64, i64]
    lib.gemvtile_gemm_splitk_splits.restype = c_int
    lib.gemvtile_gemm_splitk_workspace.argtypes = [i64, i64, i64, i64]
    lib.gemvtile_gemm_splitk_workspace.restype = i64
    lib.gemm_bf16.argtypes = [vp, vp, vp, i64, i64, i64, vp]
    lib.gemm_bf16.restype = c_int
    lib.gemv_bf16.argtypes = [vp, vp, vp, i64, i64, vp]
    lib.gemv_bf16.restype = c_int
    lib.gemvtile_gemm_f16_variant.argtypes = [vp, vp, vp, i64, i64, i64, vp, c_int]
    lib.gemvtile_gemm_f16_variant.restype = c_int
    lib.gemvtile_gemv_f16_variant.argtypes = [vp, vp, vp, i64, i64, vp, c_int]
    lib.gemvtile_gemv_f16_variant.restype = c_int
    lib.gemvtile_status_string.argtypes = [c_int]
    lib.gemvtile_status_string.restype = ctypes.c_char_p
    lib.gemvtile_tile_coord.argtypes = [i64, i64, i64, i64, i64p, i64p]
    lib.gemvtile_tile_coord.restype = c_int
    lib.gemvtile_xcd_logical_id.argtypes = [i64, i64]
    lib.gemvtile_xcd_logical_id.restype = i64
    lib.gemvtile_gemm_config.argtypes = [intp] * 6
    lib.gemvtile_gemm_config.restype = None
    lib.gemvtile_gemm_grid.argtypes = [i64, i64, i64, i64]
    lib.gemvtile_gemm_grid.restype = i64
    lib.gemvtile_gemm_tile.argtypes = [i64, i64, i64, intp, intp, intp]
    lib.gemvtile_gemm_tile.restype = c_int
    lib.gemvtile_gemv_grid.argtypes = [i64, i64, i64]
    lib.gemvtile_gemv_grid.restype = i64
    lib.gemvtile_device_caps.argtypes = [intp] * 4
    lib.gemvtile_device_caps.restype = c_int
    lib.gemvtile_ring_trace.argtypes = [c_int, i64, ctypes.POINTER(ctypes.c_int32), i64, intp]
    lib.gemvtile_ring_trace.restype = i64
    if path == LIBRARY_PATH:
        _lib = lib
    return lib


def status_string(status: int) -> str:
    return load_library().gemvtile_status_string(int(status)).decode()


def _check(status: int) -> None:
    if status != 0:
        raise GemvTileError(status, status_string(status))


# ---- raw-pointer entry points (same names and arguments as the C ABI) ------
def gemm_f16_ptr(A: int, B: int, D: int, M: int, N: int, K: int, stream: int = 0) -> int:
    """Call gemm_f16 with raw device pointers; returns the status code."""
    return int(load_library().gemm_f16(A, B, D, M, N, K, stream))


def gemv_f16_ptr(x: int, W: int, y: int, N: int, K: int, stream: int = 0) -> int:
    """Call gemv_f16 with raw device pointers; returns the status code."""
    return int(load_library().gemv_f16(x, W, y, N, K, stream))


def gemm_bf16_ptr(A: int, B: int, D: int, M: int, N: int, K: int, stream: int = 0) -> int:
    """Call gemm_bf16 with raw device pointers; returns the status code."""
    return int(load_library().gemm_bf16(A, B, D, M, N, K, stream))


def gemv_bf16_ptr(x: int, W: int, y: int, N: int, K: int, stream: int = 0) -> int:
    """Call gemv_bf16 with raw device pointers; returns the status code."""
    return int(load_library().gemv_bf16(x, W, y, N, K, stream))


# ---- tensor entry points ---------------------------------------------------
def _torch():
    import torch

    return torch


def _require(t, name, ndim, dtype=None):
    torch = _torch()
    dtype = torch.float16 if dtype is None else dtype
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (row-major)")


def _stream_handle(t, stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream(t.device).cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _gemm(A, B, D, stream, dtype, call):
    torch = _torch()
    _require(A, "A", 2, dtype)
    _require(B, "B", 2, dtype)
    M, K = A.shape
    N, K2 = B.shape
    if K != K2:
        raise ValueError(f"K mismatch: A is {tuple(A.shape)}, B is {tuple(B.shape)}")
    if B.device != A.device:
        raise ValueError("A and B must be on the same device")
    if D is None:
        D = torch.empty((M, N), dtype=dtype, device=A.device)
    else:
        _require(D, "D", 2, dtype)
        if tuple(D.shape) != (M, N) or D.device != A.device:
            raise ValueError(f"D must be [{M},{N}] on {A.device}, got {tuple(D.shape)} on {D.device}")
    s = _stream_handle(A, stream)
    with torch.cuda.device(A.device):
        st = call(A.data_ptr(), B.data_ptr(), D.data_ptr(), M, N, K, s)
    _check(st)
    return D


def gemm_f16(A, B, D=None, stream=None, variant: int = 0):
    """D = A · Bᵀ on the device.  A [M,K], B [N,K], D [M,N] fp16 contiguous.

    Enqueued on `stream` (default: the current stream) and not synchronised.
    """
    lib = load_library()
    if variant == 0:
        call = lib.gemm_f16
    else:
        def call(*args):
            return lib.gemvtile_gemm_f16_variant(*args, variant)
    return _gemm(A, B, D, stream, _torch().float16, call)


def gemm_bf16(A, B, D=None, stream=None):
    """D = A · Bᵀ on the device.  A [M,K], B [N,K], D [M,N] bfloat16 contiguous.

    Enqueued on `stream` (default: the current stream) and not synchronised.
    """
    return _gemm(A, B, D, stream, _torch().bfloat16, load_library().gemm_bf16)


# Activation codes of gemm_bias_* (gemvtile_act in gemvtile.h).
ACT_NONE = 0
ACT_RELU = 1


def _gemm_bias(A, B, bias, act, D, stream, dtype, call):
    torch = _torch()
    if isinstance(act, str):
        act = {"none": ACT_NONE, "relu": ACT_RELU}[act]
    N = B.shape[0] if isinstance(B, torch.Tensor) and B.dim() == 2 else None
    if bias is not None:
        _require(bias, "bias", 1, dtype)
        if N is not None and bias.shape[0] != N:
            raise ValueError(f"bias must have {N} elements, got {tuple(bias.shape)}")
        if bias.device != A.device:
            raise ValueError("bias must be on the device of A")
    bias_ptr = None if bias is None else bias.data_ptr()

    def with_bias(a, b, d, M, N, K, s):
        return call(a, b, bias_ptr, d, M, N, K, int(act), s)

    return _gemm(A, B, D, stream, dtype, with_bias)


def gemm_bias_f16(A, B, bias=None, act=ACT_NONE, D=None, stream=None):
    """D = act(A · Bᵀ + bias) on the device, one fp16 rounding.  A [M,K],
    B [N,K], bias [N] (or None), D [M,N] fp16 contiguous; act "none"/"relu"
    (or ACT_NONE / ACT_RELU).  Enqueued on `stream`, not synchronised."""
    return _gemm_bias(A, B, bias, act, D, stream, _torch().float16, load_library().gemm_bias_f16)


def gemm_bias_bf16(A, B, bias=None, act=ACT_NONE, D=None, stream=None):
    """gemm_bias_f16 on bfloat16 tensors."""
    return _gemm_bias(A, B, bias, act, D, stream, _torch().bfloat16, load_library().gemm_bias_bf16)


def splitk_splits(M: int, N: int, K: int, num_cus: int) -> int:
    """K slices gemm_splitk_* uses for M x N x K on num_cus CUs (1: no split)."""
    return int(load_library().gemvtile_gemm_splitk_splits(M, N, K, num_cus))


def splitk_workspace_bytes(M: int, N: int, K: int, num_cus: int) -> int:
    """Workspace bytes gemm_splitk_* needs (0 when it does not split)."""
    return int(load_library().gemvtile_gemm_splitk_workspace(M, N, K, num_cus))


def alloc_splitk_workspace(A, B, dtype=None):
    """Allocate (on the caller's behalf, explicitly) a device workspace large
    enough for gemm_splitk_*(A, B): a uint8 tensor of
    max(splitk_workspace_bytes(M, N, K, #CUs), 16) bytes on A's device.  The
    split-K calls themselves never allocate: the caller passes this (or any
    large enough) buffer as `workspace`."""
    torch = _torch()
    M, K = A.shape
    N = B.shape[0]
    cus = torch.cuda.get_device_properties(A.device).multi_processor_count
    need = splitk_workspace_bytes(M, N, K, cus)
    return torch.empty((max(need, 16),), dtype=torch.uint8, device=A.device)


def _gemm_splitk(A, B, D, workspace, stream, dtype, call):
    torch = _torch()
    if workspace is not None and (not isinstance(workspace, torch.Tensor) or not workspace.is_cuda):
        raise TypeError("workspace must be a device tensor (see alloc_splitk_workspace)")
    ws_ptr = None if workspace is None else workspace.data_ptr()
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()

    def with_ws(a, b, d, M, N, K, s):
        return call(a, b, d, M, N, K, ws_ptr, ws_bytes, s)

    return _gemm(A, B, D, stream, dtype, with_ws)


def gemm_splitk_f16(A, B, D=None, workspace=None, stream=None):
    """D = A · Bᵀ with K split across workgroups for small outputs; fp16.
    `workspace`: a device tensor of at least splitk_workspace_bytes(...)
    bytes (alloc_splitk_workspace makes one), owned by the caller.  Shapes
    that do not split need none; a shape that splits with no workspace, or
    too small a one, raises GemvTileError (GEMVTILE_ERR_INVALID_ARG).  This
    call allocates nothing but the output D when D is None.  Enqueued on
    `stream`, not synchronised."""
    return _gemm_splitk(A, B, D, workspace, stream, _torch().float16, load_library().gemm_splitk_f16)


def gemm_splitk_bf16(A, B, D=None, workspace=None, stream=None):
    """gemm_splitk_f16 on bfloat16 tensors."""
    return _gemm_splitk(A, B, D, workspace, stream, _torch().bfloat16, load_library().gemm_splitk_bf16)


def gemm_splitk_f16_noalloc(A, B, D, stream=None):
    """gemm_splitk_f16 without a workspace: the partial sums go to the
    library's static 16 MiB scratch on the device (GemvTileError with
    GEMVTILE_ERR_SCRATCH when a shape needs more).  D must be given: this
    call allocates nothing.  Calls overlapping on one GPU race; order them
    on one stream.  Enqueued on `stream`, not synchronised."""
    if D is None:
        raise ValueError("gemm_splitk_f16_noalloc allocates nothing: pass the output D")
    return _gemm(A, B, D, stream, _torch().float16, load_library().gemm_splitk_f16_noalloc)


def _gemv(x, W, y, stream, dtype, call):
    torch = _torch()
    _require(x, "x", 1, dtype)
    _require(W, "W", 2, dtype)
    N, K = W.shape
    if x.shape[0] != K:
        raise ValueError(f"K mismatch: x is {tuple(x.shape)}, W is {tuple(W.shape)}")
    if W.device != x.device:
        raise ValueError("x and W must be on the same device")
    if y is None:
        y = torch.empty((N,), dtype=dtype, device=x.device)
    else:
        _require(y, "y", 1, dtype)
        if y.shape[0] != N or y.device != x.device:
            raise ValueError(f"y must be [{N}] on {x.device}")
    s = _stream_handle(x, stream)
    with torch.cuda.device(x.device):
        st = call(x.data_ptr(), W.data_ptr(), y.data_ptr(), N, K, s)
    _check(st)
    return y


def gemv_f16(x, W, y=None, stream=None, variant: int = 0):
    """y = x · Wᵀ on the device.  x [K], W [N,K], y [N] fp16 contiguous."""
    lib = load_library()
    if variant == 0:
        call = lib.gemv_f16
    else:
        def call(*args):
            return lib.gemvtile_gemv_f16_variant(*args, variant)
    return _gemv(x, W, y, stream, _torch().float16, call)


def gemv_bf16(x, W, y=None, stream=None):
    """y = x · Wᵀ on the device.  x [K], W [N,K], y [N] bfloat16 contiguous."""
    return _gemv(x, W, y, stream, _torch().bfloat16, load_library().gemv_bf16)


def gemm_f16_variant(A, B, variant: int, D=None, stream=None):
    """gemm_f16 through an internal kernel variant (measurement only)."""
    return gemm_f16(A, B, D, stream, variant)


def gemv_f16_variant(x, W, variant: int, y=None, stream=None):
    """gemv_f16 through an internal launch shape (measurement only)."""
    return gemv_f16(x, W, y, stream, variant)


# ---- host-only helpers -----------------------------------------------------
def tile_coord(t: int, tiles_m: int, tiles_n: int, group_m: int):
    tm, tn = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().gemvtile_tile_coord(t, tiles_m, tiles_n, group_m, ctypes.byref(tm), ctypes.byref(tn)))
    return tm.value, tn.value


def xcd_logical_id(w: int, grid: int) -> int:
    return int(load_library().gemvtile_xcd_logical_id(w, grid))


def gemm_config() -> dict:
    vals = [ctypes.c_int() for _ in range(6)]
    load_library().gemvtile_gemm_config(*[ctypes.byref(v) for v in vals])
    keys = ("BM", "BN", "BK", "stages", "threads", "group_m")
    return {k: v.value for k, v in zip(keys, vals)}


def gemm_grid(M: int, N: int, K: int, num_cus: int) -> int:
    return int(load_library().gemvtile_gemm_grid(M, N, K, num_cus))


def gemm_tile(M: int, N: int, num_cus: int) -> tuple:
    """(bm, bn, stages) of the tiled GEMM for an M x N output on num_cus CUs."""
    vals = [ctypes.c_int() for _ in range(3)]
    _check(load_library().gemvtile_gemm_tile(M, N, num_cus, *[ctypes.byref(v) for v in vals]))
    return tuple(v.value for v in vals)


def gemv_grid(N: int, K: int, num_cus: int) -> int:
    return int(load_library().gemvtile_gemv_grid(N, K, num_cus))


RING_EVENTS = {1: "load", 2: "wait", 3: "lds_wait", 4: "barrier", 5: "read", 6: "mfma", 7: "prep", 8: "init"}


def ring_trace(variant: int, ktu: int):
    """The K-loop schedule of tiled GEMM variant `variant` over ktu K tiles
    (host-only): (events, info) with events a list of (name, a, b, c, d)
    tuples as gemvtile_ring_trace describes, info = {"loads_per_tile",
    "reads_per_step", "ksteps", "mfma_per_step", "stages", "bm", "bn",
    "early_free", "waves_m", "waves_n"}."""
    lib = load_library()
    info = (ctypes.c_int * 10)()
    n = int(lib.gemvtile_ring_trace(variant, ktu, None, 0, info))
    if n < 0:
        raise GemvTileError(1, f"tiled variant {variant} has no multi-stage ring, or ktu is out of range")
    buf = (ctypes.c_int32 * (5 * max(n, 1)))()
    n2 = int(lib.gemvtile_ring_trace(variant, ktu, buf, n, info))
    assert n2 == n
    events = [(RING_EVENTS[buf[5 * i]], buf[5 * i + 1], buf[5 * i + 2], buf[5 * i + 3], buf[5 * i + 4]) for i in range(n)]
    keys = ("loads_per_tile", "reads_per_step", "ksteps", "mfma_per_step", "stages", "bm", "bn", "early_free",
            "waves_m", "waves_n")
    return events, dict(zip(keys, list(info)))


def device_caps() -> dict:
    """Compute units, peak engine clock and memory clock (kHz) and memory bus
    width (bits) of the current device."""
    vals = [ctypes.c_int() for _ in range(4)]
    _check(load_library().gemvtile_device_caps(*[ctypes.byref(v) for v in vals]))
    keys = ("num_cus", "clock_khz", "mem_clock_khz", "mem_bus_bits")
    return {k: v.value for k, v in zip(keys, vals)}
