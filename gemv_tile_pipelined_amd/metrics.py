"""Algorithmic work, traffic and peaks used by the benchmark's roofline.

Counts are algorithmic, not hardware counters: the GEMV reads every element
of W once and x and y once ("Learning TileLang with GEMV", §02 Bandwidth
Bound, Table 1: 117,477,376 bytes for N = 4096, K = 14336), and the GEMM does
2·M·N·K flops on the true (unpadded) sizes.
"""
from __future__ import annotations

FP16_BYTES = 2

# MI355X published peaks (dense, no sparsity).
PEAK_HBM_GBPS = 8000.0  # 8 TB/s HBM3E
PEAK_FP16_MFMA_TFLOPS = 2500.0  # dense fp16 matrix-core peak (about 2.5 PFLOP/s)
PEAK_BF16_MFMA_TFLOPS = 2500.0  # dense bf16 matrix-core peak (same rate as fp16)
NUM_CUS = 256
ENGINE_CLOCK_GHZ = 2.4


def gemm_flops(M: int, N: int, K: int) -> int:
    """Multiply-adds of D = A·Bᵀ, two flops each."""
    return 2 * M * N * K


def gemm_bytes(M: int, N: int, K: int) -> int:
    """Compulsory HBM traffic of the GEMM: A and B read once, D written once."""
    return FP16_BYTES * (M * K + N * K + M * N)


def gemv_flops(N: int, K: int) -> int:
    return 2 * N * K


def gemv_bytes(N: int, K: int) -> int:
    """W, x read once and y written once, fp16."""
    return FP16_BYTES * (N * K + K + N)


def gemv_elements(N: int, K: int) -> dict:
    return {"W": N * K, "x": K, "y": N, "total": N * K + K + N}
