"""Kernel-trace sweep of the bandwidth-bound paths over shapes.

    rocprofv3 --kernel-trace --output-format csv -d OUT -o sweep -- \\
        python3 -m gemv_tile_pipelined_amd.shape_sweep [--gemv N:K,...] [--skinny M:N:K,...]
            [--gemm M:N:K,...] [--gemv-variants 0,8] [--skinny-variants 0,25]
            [--gemm-variants 0,53] [--gemm-data uniform,zero] [--rounds 1] [--warmup-s 1] [--gemm-bias] [--gemm-splitk]
            [--stream MB --stream-policies 1,2] [--vendor] [--reps 40] > OUT/log.txt
    python3 -m gemv_tile_pipelined_amd.shape_sweep --parse OUT OUT/log.txt

The first command launches, for every shape, `reps` GEMVs (gemv_f16, one
line per launch shape in --gemv-variants) or decode-batch GEMMs (gemm_f16,
one line per gemvtile_gemm_f16_variant id in --skinny-variants)
over enough distinct copies of W / B (at least 600 MB in all) that each
launch reads its matrix from HBM rather than the 256 MB MALL; with --vendor
also torch.mv / torch.matmul on the same inputs.  --gemm shapes run the
compute-bound GEMM (gemm_f16 through each id in --gemm-variants) over 3
rotating input sets and report TFLOP/s (2·M·N·K flops); --gemm-data picks
their values: uniform (U(-1,1) fp16, the default), m7 (the same with the
fp16 mantissa cut to its top 7 bits, bf16's precision), int (integers in
[-8, 8]) or zero, to show how the operands' bit activity moves the
power-limited clock; --rounds repeats the variant list that many times,
interleaved, so that a slow drift of the clock does not favour one variant
(--gemm-bias adds gemm_bias_f16 with a bias and ReLU to each round,
--gemm-splitk gemm_splitk_f16 with a preallocated workspace, also to the
--skinny shapes),
and the parse also prints each variant's median over the rounds.  Before
the first segment, --warmup-s seconds of untimed 4096^3 GEMMs let the clock
settle.  --stream MB runs
the read-only probe (gemvtile_read_stream, 256 workgroups) over that many MB
per launch with each cache policy in --stream-policies: the practical read
ceiling of the bandwidth-bound kernels.  Segments are delimited in the trace
by a marker kernel (a bitwise not of one int8), and the last stdout line
lists the segments.  The second command reads the trace and prints each
segment's median kernel time (summed over the kernels of one call) and
algorithmic bandwidth (2·(rows·K + K + rows) bytes for the GEMV, 2·(M·K + N·K + M·N) for the GEMM).
Inputs are seeded synthetic fp16 values (x, A ~ U(-1,1); W, B ~ U(-0.05,0.05)).
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

MARKER = "bitwise_not"
DEFAULT_GEMV = "64:14336,128:14336,256:14336,512:14336,1024:14336,2048:14336,4096:14336,1024:4096,4096:4096,256:65536,1024:65536"
DEFAULT_SKINNY = "8:256:14336,8:1024:14336,8:4096:14336,8:1024:4096"


def _shapes(spec, n):
    out = []
    for item in filter(None, spec.split(",")):
        vals = tuple(int(v) for v in item.split(":"))
        if len(vals) != n:
            raise SystemExit(f"shape {item!r}: expected {n} sizes")
        out.append(vals)
    return out


def run(a):
    import torch

    import gemv_tile_pipelined_amd as gt

    dev = torch.device("cuda:0")
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    marker = torch.zeros((1,), dtype=torch.int8, device=dev)
    labels = []

    def copies_for(nbytes):
        return max(2, min(64, int(600e6 // nbytes) + 1))

    def segment(label, fn, copies):
        try:
            fn(0)
        except gt.GemvTileError as e:
            if e.status != 2:  # only launch shapes that do not apply to this shape are skipped
                raise
            return
        for i in range(1, 3):
            fn(i % copies)
        torch.cuda.synchronize(dev)
        marker.bitwise_not_()
        for i in range(a.reps):
            fn(i % copies)
        marker.bitwise_not_()
        torch.cuda.synchronize(dev)
        labels.append(label)

    def uni(shape, lo, hi):
        return torch.empty(shape, dtype=torch.float16, device=dev).uniform_(lo, hi, generator=g)

    if a.warmup_s > 0:
        # Untimed load before the first marker: the part's clock takes a few
        # tenths of a second of sustained work to settle, and segments run
        # before that would read slow for reasons of their position alone.
        import time

        wa, wb = uni((4096, 4096), -1, 1), uni((4096, 4096), -1, 1)
        wd = torch.empty((4096, 4096), dtype=torch.float16, device=dev)
        t_end = time.monotonic() + a.warmup_s
        while time.monotonic() < t_end:
            for _ in range(50):
                gt.gemm_f16(wa, wb, wd)
            torch.cuda.synchronize(dev)
        del wa, wb, wd

    variants = [int(v) for v in a.gemv_variants.split(",")]
    skinny_variants = [int(v) for v in a.skinny_variants.split(",")]
    for N, K in _shapes(a.gemv, 2):
        c = copies_for(2 * N * K)
        x = uni((K,), -1, 1)
        Ws = [uni((N, K), -0.05, 0.05) for _ in range(c)]
        y = torch.empty((N,), dtype=torch.float16, device=dev)
        nbytes = 2 * (N * K + N + K)
        for v in variants:
            segment({"kind": "gemv_f16", "N": N, "K": K, "variant": v, "bytes": nbytes},
                    lambda i, v=v: gt.gemv_f16(x, Ws[i], y, variant=v), c)
        if a.vendor:
            segment({"kind": "torch.mv", "N": N, "K": K, "bytes": nbytes}, lambda i: torch.mv(Ws[i], x, out=y), c)
        del Ws
    for M, N, K in _shapes(a.skinny, 3):
        c = copies_for(2 * N * K)
        A = uni((M, K), -1, 1)
        Bs = [uni((N, K), -0.05, 0.05) for _ in range(c)]
        D = torch.empty((M, N), dtype=torch.float16, device=dev)
        for v in skinny_variants:
            segment({"kind": "gemm_f16", "M": M, "N": N, "K": K, "variant": v, "bytes": 2 * (M * K + N * K + M * N)},
                    lambda i, v=v: gt.gemm_f16(A, Bs[i], D, variant=v), c)
        if a.gemm_splitk:
            cus = torch.cuda.get_device_properties(dev).multi_processor_count
            ws = torch.empty((max(gt.splitk_workspace_bytes(M, N, K, cus), 16),), dtype=torch.uint8, device=dev)
            segment({"kind": "gemm_splitk", "M": M, "N": N, "K": K, "bytes": 2 * (M * K + N * K + M * N)},
                    lambda i: gt.gemm_splitk_f16(A, Bs[i], D, workspace=ws), c)
        if a.vendor:
            segment({"kind": "torch.matmul", "M": M, "N": N, "K": K, "bytes": 2 * (M * K + N * K + M * N)},
                    lambda i: torch.matmul(A, Bs[i].t(), out=D), c)
        del Bs
    if a.stream > 0:
        nbytes = int(a.stream * 1e6) // 16 * 16
        c = copies_for(nbytes)
        bufs = [uni((nbytes // 2,), -1, 1) for _ in range(c)]
        sink = torch.zeros((256,), dtype=torch.int32, device=dev)
        for pol in [int(v) for v in a.stream_policies.split(",")]:
            segment({"kind": "read_stream", "policy": pol, "N": nbytes, "bytes": nbytes},
                    lambda i, pol=pol: gt.read_stream(bufs[i], sink, pol, 256), c)
        del bufs
    def operand(shape, data):
        if data == "uniform":
            return uni(shape, -1, 1)
        if data == "m7":  # keep the top 7 of fp16's 10 mantissa bits
            t = uni(shape, -1, 1)
            return (t.view(torch.int16) & ~0x7).view(torch.float16)
        if data == "int":
            return torch.randint(-8, 9, shape, device=dev, generator=g).to(torch.float16)
        if data == "zero":
            return torch.zeros(shape, dtype=torch.float16, device=dev)
        raise SystemExit(f"unknown --gemm-data {data!r}")

    gemm_variants = [int(v) for v in a.gemm_variants.split(",")]
    for M, N, K in _shapes(a.gemm, 3):
        for data in a.gemm_data.split(","):
            sets = [(operand((M, K), data), operand((N, K), data)) for _ in range(3)]
            D = torch.empty((M, N), dtype=torch.float16, device=dev)
            bias = uni((N,), -4, 4)
            cus = torch.cuda.get_device_properties(dev).multi_processor_count
            ws = torch.empty((max(gt.splitk_workspace_bytes(M, N, K, cus), 16),), dtype=torch.uint8, device=dev)
            for rnd in range(a.rounds):
                for v in gemm_variants:
                    segment({"kind": "gemm_f16", "M": M, "N": N, "K": K, "variant": v, "data": data,
                             "round": rnd, "flops": 2 * M * N * K},
                            lambda i, v=v: gt.gemm_f16(sets[i][0], sets[i][1], D, variant=v), 3)
                if a.gemm_splitk:
                    segment({"kind": "gemm_splitk", "M": M, "N": N, "K": K, "data": data, "round": rnd,
                             "flops": 2 * M * N * K},
                            lambda i: gt.gemm_splitk_f16(sets[i][0], sets[i][1], D, workspace=ws), 3)
                if a.gemm_bias:
                    segment({"kind": "gemm_bias", "M": M, "N": N, "K": K, "data": data, "round": rnd,
                             "flops": 2 * M * N * K},
                            lambda i: gt.gemm_bias_f16(sets[i][0], sets[i][1], bias, gt.ACT_RELU, D), 3)
                if a.vendor:
                    segment({"kind": "torch.matmul", "M": M, "N": N, "K": K, "data": data, "round": rnd,
                             "flops": 2 * M * N * K},
                            lambda i: torch.matmul(sets[i][0], sets[i][1].t(), out=D), 3)
            del sets
    print("SEGMENTS " + json.dumps(labels), flush=True)


def parse(trace_dir, log_path):
    trace = sorted(glob.glob(os.path.join(trace_dir, "**", "*kernel_trace.csv"), recursive=True))
    if not trace:
        raise SystemExit(f"no kernel_trace.csv under {trace_dir}")
    labels = None
    for line in open(log_path):
        if line.startswith("SEGMENTS "):
            labels = json.loads(line[len("SEGMENTS "):])
    if labels is None:
        raise SystemExit(f"no SEGMENTS line in {log_path}")
    rows = sorted(csv.DictReader(open(trace[0])), key=lambda r: int(r["Start_Timestamp"]))
    marks = [i for i, r in enumerate(rows) if MARKER in r["Kernel_Name"]]
    if len(marks) != 2 * len(labels):
        raise SystemExit(f"{len(marks)} markers for {len(labels)} segments")
    by_label: dict = {}
    for lab, (lo, hi) in zip(labels, zip(marks[0::2], marks[1::2])):
        # A call may launch several kernels (split K: the partial GEMM, then
        # the reduction): the segment's time per call is the sum over kernel
        # names of each one's median duration.
        per_kernel: dict = {}
        for r in rows[lo + 1 : hi]:
            per_kernel.setdefault(r["Kernel_Name"].split("(")[0][:60], []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
        names = sorted(per_kernel)
        durs = per_kernel[names[0]] if names else []
        kmeds = {n: statistics.median(d) / 1e3 for n, d in per_kernel.items()}
        med = sum(kmeds.values())
        if len(kmeds) > 1:
            names = [f"{n} {kmeds[n]:.2f} us" for n in names]
        shape = "x".join(str(lab[k]) for k in ("M", "N", "K") if k in lab)
        var = f" v{lab['variant']}" if "variant" in lab else (f" p{lab['policy']}" if "policy" in lab else "")
        if "data" in lab:
            shape += f" {lab['data']}"
        if "flops" in lab:
            tf = lab["flops"] / (med * 1e6)
            rate = f"{tf:6.0f} TFLOP/s ({tf / 25:5.1f} % of 2.5 PFLOP/s)"
        else:
            gbps = lab["bytes"] / (med * 1e3)
            rate = f"{gbps:6.0f} GB/s ({gbps / 80:5.1f} % of 8 TB/s)"
        print(f"{lab['kind']:13s}{var:4s} {shape:18s} n={len(durs):3d} median {med:8.2f} us {rate}  {'; '.join(names)}")
        key = json.dumps({k: v for k, v in lab.items() if k != "round"}, sort_keys=True)
        by_label.setdefault(key, []).append(med)
    repeated = {k: v for k, v in by_label.items() if len(v) > 1}
    if repeated:
        print("-- over rounds: median of the segment medians (min .. max)")
        for key, meds in repeated.items():
            lab = json.loads(key)
            var = f" v{lab['variant']}" if "variant" in lab else ""
            shape = "x".join(str(lab[k]) for k in ("M", "N", "K") if k in lab) + f" {lab.get('data', '')}"
            print(f"{lab['kind']:13s}{var:4s} {shape:18s} rounds={len(meds):2d} {statistics.median(meds):8.2f} us "
                  f"({min(meds):.2f} .. {max(meds):.2f})")


def main(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gemv", default=DEFAULT_GEMV, help="N:K,... (empty for none)")
    p.add_argument("--skinny", default=DEFAULT_SKINNY, help="M:N:K,... (empty for none)")
    p.add_argument("--gemv-variants", default="0")
    p.add_argument("--skinny-variants", default="0")
    p.add_argument("--gemm", default="", help="M:N:K,... compute-bound GEMM shapes (default none)")
    p.add_argument("--gemm-variants", default="0")
    p.add_argument("--gemm-data", default="uniform", help="uniform,m7,int,zero (comma list)")
    p.add_argument("--rounds", type=int, default=1, help="times the --gemm-variants list runs, interleaved")
    p.add_argument("--gemm-bias", action="store_true", help="also gemm_bias_f16 (bias + ReLU) on each GEMM shape")
    p.add_argument("--gemm-splitk", action="store_true", help="also gemm_splitk_f16 on each GEMM shape")
    p.add_argument("--warmup-s", type=float, default=1.0, help="seconds of untimed GEMMs before the first segment")
    p.add_argument("--stream", type=float, default=0.0, help="MB per read-only probe launch (0: none)")
    p.add_argument("--stream-policies", default="1,2")
    p.add_argument("--vendor", action="store_true")
    p.add_argument("--reps", type=int, default=40)
    p.add_argument("--parse", nargs=2, metavar=("TRACE_DIR", "LOG"))
    a = p.parse_args(argv)
    if a.parse:
        parse(*a.parse)
    else:
        run(a)


if __name__ == "__main__":
    main()
