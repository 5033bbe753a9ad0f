"""Seeded synthetic inputs shared by the CPU oracle tests and the GPU path.

This module only draws numbers; it holds none of the arithmetic of the
method.  Every tensor is identified by a (config id, tensor id) pair and is
drawn from ``numpy.random.default_rng(SeedSequence([cfg_id, tensor_id]))`` as
float64 and then cast to float16 with numpy's round-to-nearest-even cast, so
that both sides of every comparison consume the same fp16 bit patterns.

Tensor ids: 0 = A (GEMM) or x (GEMV), 1 = B (GEMM) or W (GEMV),
2 = the sampled output rows of a large GEMM.  Further ids are used by the
tests for extra draws (integer-valued inputs, small shapes).

The workloads follow the pages: the GEMM is D = A·Bᵀ with A [M,K] and B [N,K]
row-major (K-contiguous), as in the TVM TIRx GEMM chapter ("使用 TMA 为 GEMM
建立 Pipeline", step 4 full kernel) and the Croqtile pipelined matmul
(ch. 7, lhs [M,K] / rhs [N,K]); the GEMV is y = x·Wᵀ with W [N,K] row-major,
N=4096, K=14336, as in "Learning TileLang with GEMV" (§01 GEMV).
"""
from __future__ import annotations

import dataclasses

import numpy as np

__all__ = [
    "Workload",
    "WORKLOADS",
    "DECODE_BATCH",
    "rng",
    "uniform_f16",
    "integer_f16",
    "uniform_bf16",
    "integer_bf16",
    "sample_rows",
    "band_rows",
    "gemm_inputs",
    "gemv_inputs",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: its shape and the value distribution."""

    cfg_id: int
    name: str
    kind: str  # "gemm" or "gemv"
    M: int  # rows of A / D (1 for the GEMV)
    N: int  # rows of B (GEMM) or W (GEMV)
    K: int  # reduction length
    lo_a: float  # uniform range of A (GEMM) or x (GEMV)
    hi_a: float
    lo_b: float  # uniform range of B (GEMM) or W (GEMV)
    hi_b: float
    sampled_rows: int = 0  # >0: compare only this many seeded output rows


# The five workloads, in a fixed order that also fixes their seeds.
WORKLOADS = (
    Workload(0, "gemm_256", "gemm", 256, 256, 256, -1.0, 1.0, -1.0, 1.0),
    Workload(1, "gemm_4096", "gemm", 4096, 4096, 4096, -1.0, 1.0, -1.0, 1.0),
    Workload(2, "gemm_ragged_4000x4032x4104", "gemm", 4000, 4032, 4104, -1.0, 1.0, -1.0, 1.0),
    Workload(3, "gemv_4096x14336", "gemv", 1, 4096, 14336, -1.0, 1.0, -0.05, 0.05),
    Workload(4, "gemm_8192", "gemm", 8192, 8192, 8192, -1.0, 1.0, -1.0, 1.0, sampled_rows=64),
)


# A decode batch: 8 activation rows against the GEMV's weight matrix shape,
# D = A·Bᵀ with A [8,14336] ~ uniform(-1,1) and B [4096,14336] ~
# uniform(-0.05,0.05) -- the GEMV workload with a batch of 8 instead of 1.
DECODE_BATCH = Workload(5, "gemm_decode_8x4096x14336", "gemm", 8, 4096, 14336, -1.0, 1.0, -0.05, 0.05)


def rng(cfg_id: int, tensor_id: int) -> np.random.Generator:
    """The generator for one tensor of one workload."""
    return np.random.default_rng(np.random.SeedSequence([int(cfg_id), int(tensor_id)]))


def uniform_f16(cfg_id: int, tensor_id: int, shape, lo: float, hi: float) -> np.ndarray:
    """uniform(lo, hi) drawn in float64, then cast to float16 (RNE)."""
    g = rng(cfg_id, tensor_id)
    return g.uniform(lo, hi, size=shape).astype(np.float16)


def integer_f16(cfg_id: int, tensor_id: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi], stored as float16 (exact)."""
    g = rng(cfg_id, tensor_id)
    return g.integers(lo, hi + 1, size=shape).astype(np.float16)


def uniform_bf16(cfg_id: int, tensor_id: int, shape, lo: float, hi: float) -> np.ndarray:
    """bf16 values as uint16 bit patterns (numpy has no bfloat16 dtype):
    uniform(lo, hi) drawn in float64, cast to float32, and the low 16 bits of
    the float32 pattern dropped (rounding toward zero, so the input draw does
    not use the method's round-to-nearest)."""
    g = rng(cfg_id, tensor_id)
    f = g.uniform(lo, hi, size=shape).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def integer_bf16(cfg_id: int, tensor_id: int, shape, lo: int = -8, hi: int = 8) -> np.ndarray:
    """Integers drawn uniformly from [lo, hi] as bf16 bit patterns (exact)."""
    g = rng(cfg_id, tensor_id)
    f = g.integers(lo, hi + 1, size=shape).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)


def sample_rows(cfg_id: int, M: int, count: int) -> np.ndarray:
    """`count` distinct row indices of [0, M), sorted (tensor id 2)."""
    g = rng(cfg_id, 2)
    return np.sort(g.choice(M, size=min(count, M), replace=False)).astype(np.int64)


def band_rows(cfg_id: int, M: int, band: int = 256) -> np.ndarray:
    """One row drawn uniformly from every `band`-row band of [0, M) (tensor
    id 4), sorted: with band = the output tile height, every tile row of the
    output holds at least one of them."""
    g = rng(cfg_id, 4)
    starts = np.arange(0, M, band)
    return np.sort(starts + np.floor(g.random(len(starts)) * np.minimum(band, M - starts)).astype(np.int64))


def gemm_inputs(w: Workload, integer: bool = False, bf16: bool = False):
    """(A, B) for a GEMM workload, each C-contiguous: float16 arrays, or bf16
    bit patterns (uint16) when `bf16` is set."""
    assert w.kind == "gemm"
    uni, intg = (uniform_bf16, integer_bf16) if bf16 else (uniform_f16, integer_f16)
    if integer:
        # Separate tensor ids (10, 11) so the integer draw never aliases the
        # uniform one.
        return (intg(w.cfg_id, 10, (w.M, w.K)), intg(w.cfg_id, 11, (w.N, w.K)))
    return (
        uni(w.cfg_id, 0, (w.M, w.K), w.lo_a, w.hi_a),
        uni(w.cfg_id, 1, (w.N, w.K), w.lo_b, w.hi_b),
    )


def gemv_inputs(w: Workload, integer: bool = False, bf16: bool = False):
    """(x, W) for a GEMV workload (float16, or bf16 bit patterns when `bf16`)."""
    assert w.kind == "gemv"
    uni, intg = (uniform_bf16, integer_bf16) if bf16 else (uniform_f16, integer_f16)
    if integer:
        return (intg(w.cfg_id, 10, (w.K,)), intg(w.cfg_id, 11, (w.N, w.K)))
    return (
        uni(w.cfg_id, 0, (w.K,), w.lo_a, w.hi_a),
        uni(w.cfg_id, 1, (w.N, w.K), w.lo_b, w.hi_b),
    )
