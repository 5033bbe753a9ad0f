"""CPU oracle for the FP16 GEMM / GEMV -- test infrastructure only.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never imports it and
it never imports the GPU library; the two share no code.

The arithmetic lives in ``oracle.c`` (plain C, FP64 accumulation, its own
IEEE binary16 conversions); this module only compiles it, loads it with
ctypes and marshals numpy arrays.  See the header of ``oracle.c`` for the
definitions and the passages of the pages they follow.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

_lib = None


def compile_oracle(source: str = SOURCE, output: str = LIBRARY, extra_flags=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", *extra_flags, source, "-o", output, "-lm"]
    subprocess.run(cmd, check=True)
    return output


def load(path: str = LIBRARY, build_if_missing: bool = True):
    """Load (and if needed compile) the oracle library; returns a ctypes CDLL."""
    global _lib
    if path == LIBRARY and _lib is not None:
        return _lib
    if not os.path.exists(path):
        if not build_if_missing:
            raise FileNotFoundError(path)
        compile_oracle(output=path)
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f64p = ctypes.POINTER(ctypes.c_double)
    i64p = ctypes.POINTER(ctypes.c_int64)
    i64 = ctypes.c_int64
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_f16_rne.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_f16_rne.restype = ctypes.c_uint16
    lib.oracle_f16_to_f64_array.argtypes = [u16p, f64p, i64]
    lib.oracle_f16_to_f64_array.restype = None
    lib.oracle_f64_to_f16_array.argtypes = [f64p, u16p, i64]
    lib.oracle_f64_to_f16_array.restype = None
    lib.oracle_gemm_f16.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64p, i64, ctypes.c_int]
    lib.oracle_gemm_f16.restype = ctypes.c_int
    lib.oracle_gemv_f16.argtypes = [u16p, u16p, u16p, i64, i64, ctypes.c_int]
    lib.oracle_gemv_f16.restype = ctypes.c_int
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_bf16_rne.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16_rne.restype = ctypes.c_uint16
    lib.oracle_bf16_to_f64_array.argtypes = [u16p, f64p, i64]
    lib.oracle_bf16_to_f64_array.restype = None
    lib.oracle_f64_to_bf16_array.argtypes = [f64p, u16p, i64]
    lib.oracle_f64_to_bf16_array.restype = None
    lib.oracle_gemm_bf16.argtypes = [u16p, u16p, u16p, i64, i64, i64, i64p, i64, ctypes.c_int]
    lib.oracle_gemm_bf16.restype = ctypes.c_int
    lib.oracle_gemv_bf16.argtypes = [u16p, u16p, u16p, i64, i64, ctypes.c_int]
    lib.oracle_gemv_bf16.restype = ctypes.c_int
    lib.oracle_gemm_bias_f16.argtypes = [u16p, u16p, u16p, ctypes.c_int, u16p, i64, i64, i64, i64p, i64, ctypes.c_int]
    lib.oracle_gemm_bias_f16.restype = ctypes.c_int
    lib.oracle_gemm_bias_bf16.argtypes = [u16p, u16p, u16p, ctypes.c_int, u16p, i64, i64, i64, i64p, i64, ctypes.c_int]
    lib.oracle_gemm_bias_bf16.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    lib.oracle_max_threads.restype = ctypes.c_int
    if path == LIBRARY:
        _lib = lib
    return lib


def _u16(a: np.ndarray):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.float16, a.dtype
    return a.view(np.uint16), a.view(np.uint16).ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def f16_to_f64(h: np.ndarray, lib=None) -> np.ndarray:
    """Decode float16 values (or raw uint16 bit patterns) to float64."""
    lib = lib or load()
    bits = np.ascontiguousarray(h).view(np.uint16).ravel()
    out = np.empty(bits.shape, np.float64)
    lib.oracle_f16_to_f64_array(
        bits.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        bits.size,
    )
    return out.reshape(np.shape(h))


def f64_to_f16(v: np.ndarray, lib=None) -> np.ndarray:
    """Round float64 values to float16 (nearest, ties to even)."""
    lib = lib or load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    flat = v.ravel()
    out = np.empty(flat.shape, np.uint16)
    lib.oracle_f64_to_f16_array(
        flat.ctypes.data_as(ctypes.POINTER(ctypes.c_double)),
        out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)),
        flat.size,
    )
    return out.view(np.float16).reshape(v.shape)


def gemm(A: np.ndarray, B: np.ndarray, rows=None, nthreads: int = 0, lib=None) -> np.ndarray:
    """D = A·Bᵀ in FP64, rounded once to fp16.  ``rows`` selects output rows."""
    lib = lib or load()
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    _, pa = _u16(A)
    _, pb = _u16(B)
    if rows is None:
        nrows = M
        prow = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows.size
        prow = rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    D = np.empty((nrows, N), np.float16)
    _, pd = _u16(D)
    rc = lib.oracle_gemm_f16(pa, pb, pd, M, N, K, prow, nrows, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemm_f16 failed ({rc})")
    return D


def gemv(x: np.ndarray, W: np.ndarray, nthreads: int = 0, lib=None) -> np.ndarray:
    """y = x·Wᵀ in FP64, rounded once to fp16."""
    lib = lib or load()
    N, K = W.shape
    assert x.shape == (K,)
    _, px = _u16(x)
    _, pw = _u16(W)
    y = np.empty((N,), np.float16)
    _, py = _u16(y)
    rc = lib.oracle_gemv_f16(px, pw, py, N, K, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemv_f16 failed ({rc})")
    return y


# ---- bf16: numpy has no bfloat16 dtype, so bf16 arrays are uint16 bit patterns
def _bf16_bits(a: np.ndarray):
    a = np.ascontiguousarray(a)
    assert a.dtype == np.uint16, f"bf16 arrays are passed as uint16 bit patterns, got {a.dtype}"
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16))


def bf16_to_f64(bits: np.ndarray, lib=None) -> np.ndarray:
    """Decode bf16 bit patterns (uint16) to float64."""
    lib = lib or load()
    b = np.ascontiguousarray(bits, dtype=np.uint16).ravel()
    out = np.empty(b.shape, np.float64)
    lib.oracle_bf16_to_f64_array(
        b.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), out.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), b.size
    )
    return out.reshape(np.shape(bits))


def f64_to_bf16(v: np.ndarray, lib=None) -> np.ndarray:
    """Round float64 values to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    lib = lib or load()
    v = np.ascontiguousarray(v, dtype=np.float64)
    flat = v.ravel()
    out = np.empty(flat.shape, np.uint16)
    lib.oracle_f64_to_bf16_array(
        flat.ctypes.data_as(ctypes.POINTER(ctypes.c_double)), out.ctypes.data_as(ctypes.POINTER(ctypes.c_uint16)), flat.size
    )
    return out.reshape(v.shape)


def gemm_bf16(A: np.ndarray, B: np.ndarray, rows=None, nthreads: int = 0, lib=None) -> np.ndarray:
    """D = A·Bᵀ for bf16 bit arrays, in FP64, rounded once to bf16 (bit patterns out)."""
    lib = lib or load()
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    _, pa = _bf16_bits(A)
    _, pb = _bf16_bits(B)
    if rows is None:
        nrows, prow = M, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, prow = rows.size, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    D = np.empty((nrows, N), np.uint16)
    _, pd = _bf16_bits(D)
    rc = lib.oracle_gemm_bf16(pa, pb, pd, M, N, K, prow, nrows, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemm_bf16 failed ({rc})")
    return D


def gemv_bf16(x: np.ndarray, W: np.ndarray, nthreads: int = 0, lib=None) -> np.ndarray:
    """y = x·Wᵀ for bf16 bit arrays, in FP64, rounded once to bf16 (bit patterns out)."""
    lib = lib or load()
    N, K = W.shape
    assert x.shape == (K,)
    _, px = _bf16_bits(x)
    _, pw = _bf16_bits(W)
    y = np.empty((N,), np.uint16)
    _, py = _bf16_bits(y)
    rc = lib.oracle_gemv_bf16(px, pw, py, N, K, int(nthreads))
    if rc != 0:
        raise ValueError(f"oracle_gemv_bf16 failed ({rc})")
    return y


ACT_NONE = 0
ACT_RELU = 1


def _gemm_bias(fname, to_bits, dtype, A, B, bias, act, rows, nthreads, lib):
    lib = lib or load()
    M, K = A.shape
    N, K2 = B.shape
    assert K == K2
    # keep the (possibly copied) contiguous arrays alive while C reads them
    a_arr, pa = to_bits(A)
    b_arr, pb = to_bits(B)
    bias_arr, pbias = (None, None) if bias is None else to_bits(bias)
    assert bias is None or np.shape(bias) == (N,)
    if rows is None:
        nrows, prow = M, None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        nrows, prow = rows.size, rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    D = np.empty((nrows, N), dtype)
    _, pd = to_bits(D)
    rc = getattr(lib, fname)(pa, pb, pbias, int(act), pd, M, N, K, prow, nrows, int(nthreads))
    if rc != 0:
        raise ValueError(f"{fname} failed ({rc})")
    return D


def gemm_bias(A: np.ndarray, B: np.ndarray, bias=None, act: int = ACT_NONE, rows=None, nthreads: int = 0,
              lib=None) -> np.ndarray:
    """D = act(A·Bᵀ + bias) in FP64 (bias [N] added to every row, act
    ACT_NONE or ACT_RELU), rounded once to fp16."""
    return _gemm_bias("oracle_gemm_bias_f16", _u16, np.float16, A, B, bias, act, rows, nthreads, lib)


def gemm_bias_bf16(A: np.ndarray, B: np.ndarray, bias=None, act: int = ACT_NONE, rows=None, nthreads: int = 0,
                   lib=None) -> np.ndarray:
    """gemm_bias for bf16 bit arrays (uint16 in and out)."""
    return _gemm_bias("oracle_gemm_bias_bf16", _bf16_bits, np.uint16, A, B, bias, act, rows, nthreads, lib)


def max_threads(lib=None) -> int:
    lib = lib or load()
    return int(lib.oracle_max_threads())
