"""Run one kernel of the library a few times, for hardware-counter profiling.

    python -m gemv_tile_pipelined_amd.profile_driver gemm [--variant V] [--shape M N K] [--iters I]
    python -m gemv_tile_pipelined_amd.profile_driver gemv [--variant V] [--shape N K] [--iters I]
    python -m gemv_tile_pipelined_amd.profile_driver decode [--variant V] [--shape M N K] [--iters I]
    python -m gemv_tile_pipelined_amd.profile_driver copy [--mib S] [--iters I]

`--bf16` runs gemm_bf16 / gemv_bf16 on bf16 inputs of the same shapes instead
(default kernels only).  For `gemm`, `--data zero|int` replaces the uniform
operands (zeros, or integers in [-8, 8]: fewer active bits, less power) and
`--vendor` runs torch.matmul on the same operands instead of the library.

Meant to run under `rocprofv3 --pmc ...`: every dispatch of the chosen kernel
then carries its counters.  `copy` runs a plain device-to-device copy of a
known size, which calibrates byte counters (FETCH_SIZE, WRITE_SIZE) against
bytes that are known exactly.  Inputs are seeded synthetic fp16 values; the
GEMV and the decode batch (gemm_f16 with few rows of A, default 8x4096x14336)
cycle through 5 copies of W / B so every dispatch reads it from HBM.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main(argv=None):
    p = argparse.ArgumentParser()
    p.add_argument("kernel", choices=["gemm", "gemv", "decode", "copy"])
    p.add_argument("--variant", type=int, default=0)
    p.add_argument("--shape", type=int, nargs="+", default=None)
    p.add_argument("--iters", type=int, default=10)
    p.add_argument("--mib", type=int, default=512)
    p.add_argument("--bf16", action="store_true")
    p.add_argument("--data", choices=["uniform", "zero", "int"], default="uniform")
    p.add_argument("--vendor", action="store_true")
    a = p.parse_args(argv)

    import torch

    import gemv_tile_pipelined_amd as gt

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    dt = torch.bfloat16 if a.bf16 else torch.float16
    if a.bf16 and a.variant != 0:
        p.error("--bf16 runs the default kernels only")

    def gemm(A, B, D):
        if a.bf16:
            gt.gemm_bf16(A, B, D)
        else:
            gt.gemm_f16(A, B, D, variant=a.variant)

    def gemv(x, W, y):
        if a.bf16:
            gt.gemv_bf16(x, W, y)
        else:
            gt.gemv_f16(x, W, y, variant=a.variant)

    if a.kernel == "gemm":
        M, N, K = a.shape or (4096, 4096, 4096)

        def operand(rows):
            if a.data == "zero":
                return torch.zeros((rows, K), dtype=dt, device=dev)
            if a.data == "int":
                return torch.randint(-8, 9, (rows, K), device=dev, generator=g).to(dt)
            return torch.empty((rows, K), dtype=dt, device=dev).uniform_(-1, 1, generator=g)

        A, B = operand(M), operand(N)
        D = torch.empty((M, N), dtype=dt, device=dev)
        for _ in range(a.iters):
            if a.vendor:
                torch.matmul(A, B.t(), out=D)
            else:
                gemm(A, B, D)
    elif a.kernel == "decode":
        M, N, K = a.shape or (8, 4096, 14336)
        A = torch.empty((M, K), dtype=dt, device=dev).uniform_(-1, 1, generator=g)
        Bs = [torch.empty((N, K), dtype=dt, device=dev).uniform_(-0.05, 0.05, generator=g) for _ in range(5)]
        D = torch.empty((M, N), dtype=dt, device=dev)
        for i in range(a.iters):
            gemm(A, Bs[i % 5], D)
    elif a.kernel == "gemv":
        N, K = a.shape or (4096, 14336)
        x = torch.empty((K,), dtype=dt, device=dev).uniform_(-1, 1, generator=g)
        Ws = [torch.empty((N, K), dtype=dt, device=dev).uniform_(-0.05, 0.05, generator=g) for _ in range(5)]
        y = torch.empty((N,), dtype=dt, device=dev)
        for i in range(a.iters):
            gemv(x, Ws[i % 5], y)
    else:
        n = a.mib * 1024 * 1024 // 2
        src = torch.empty((n,), dtype=torch.float16, device=dev).uniform_(-1, 1, generator=g)
        dst = torch.empty_like(src)
        for _ in range(a.iters):
            dst.copy_(src)
    torch.cuda.synchronize(dev)
    print(f"profile_driver {a.kernel} done ({a.iters} dispatches)", flush=True)


if __name__ == "__main__":
    main()
