"""Benchmark of the FP16 GEMM / GEMV hot path on one MI355X.

One step = one gemm_f16 at M = N = K = 4096 plus five gemv_f16 at N = 4096,
K = 14336, one over each of five distinct copies of W (the whole hot path;
587 MB of W per step, more than twice the 256 MB MALL, so every GEMV streams
its W from HBM rather than from cache), on seeded synthetic fp16 inputs
already resident in device memory.  The GEMM rotates over 3 input sets.

Prints ONE JSON line on stdout:
  value        GEMM TFLOP/s (2·M·N·K / mean GEMM kernel time, HIP events)
  roofline     GEMM against the dense fp16 MFMA peak
  gemv         GEMV GB/s (algorithmic bytes 2·(N·K + K + N) / mean kernel time,
               the five back-to-back launches of a step timed together)
               with its own roofline against the HBM peak
  decode_batch the 8x4096x14336 GEMM (skinny path) in GB/s, timed on its own
  bf16         gemm_bf16 at 4096^3 and gemv_bf16 at 4096x14336, bf16 inputs of
               the same shapes, timed on their own after the decode batch
  vendor_same_box  torch.matmul on the same fp16 4096^3 inputs, timed after
               the rest: where this box's power-limited clock stands
  cpu_baseline the CPU oracle (FP64, OpenMP) on a bounded sample of rows of
               the same GEMM, scaled to TFLOP/s, plus the full GEMV in GB/s
Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 2000]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fp16 GEMM TFLOP/s @4096³ (% MFMA peak); GEMV GB/s (% HBM peak)"
GEMM_M = GEMM_N = GEMM_K = 4096
GEMV_N, GEMV_K = 4096, 14336
GEMM_SETS = 3
DECODE_REPS = 20  # event pairs around 5 decode-batch launches, after the timed steps
BF16_REPS = 50  # event triples around one gemm_bf16 and 5 gemv_bf16, after the decode batch
SECTION_WARMUP = 200  # untimed repetitions before the decode-batch, bf16 and vendor timings
VENDOR_REPS = 50  # event pairs around one vendor GEMM, the same-box reference
GEMV_COPIES = 5
# Beyond-L2 traffic per launch measured with rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch, each scaled by what the same counter reads for
# a device copy of known size: x2.000 for FETCH_SIZE, x1.000 for WRITE_SIZE),
# valid only for the kernel sources whose SHA-256 is recorded here; the
# summary and commands are in profiles/traffic_fetch_write_size.md.
MEASURED_TRAFFIC = {
    "sources_sha256": "6323810194d9726681cb6e36b7babe9525dcd48328e50184f0ab574aac325c3e",
    "gemm": {"fetch_kib": 98433.6 * 2.0, "write_kib": 32792.2 * 1.0},
    "gemv": {"fetch_kib": 57475.8 * 2.0, "write_kib": 8.0 * 1.0},
    "decode": {"fetch_kib": 58257.3 * 2.0, "write_kib": 64.0 * 1.0},
    "gemm_bf16": {"fetch_kib": 98435.0 * 2.0, "write_kib": 32793.5 * 1.0},
    "gemv_bf16": {"fetch_kib": 57480.8 * 2.0, "write_kib": 8.0 * 1.0},
}
KERNEL_SOURCES = ("device_common.hpp", "gemm.hip", "gemv.hip", "kernels.hpp", "skinny.hip", "tile_order.hpp")


def kernel_sources_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gemv_tile_pipelined_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    # About 0.4 s of untimed steps: under sustained load the part's clocks take
    # a few tenths of a second to settle, and 20 warm-up steps (4 ms) left the
    # GEMM 5-7 % slower than its steady state.
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--cpu-seconds", type=float, default=12.0, help="target CPU time of the oracle sample")
    return p.parse_args()


def cpu_baseline(target_s: float):
    """The oracle as it stands, on rows of the 4096^3 GEMM and on the full GEMV."""
    import numpy as np

    import datagen
    import oracle

    lib = oracle.load()
    threads = oracle.max_threads(lib)
    w = datagen.WORKLOADS[1]
    A, B = datagen.gemm_inputs(w)
    # calibrate on 64 rows (the fixed cost of decoding B is paid in both
    # runs), then size the sample to about target_s seconds, at most the
    # whole GEMM
    rows = datagen.sample_rows(1, w.M, 64)
    oracle.gemm(A, B, rows=rows[:8], lib=lib)
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=rows, lib=lib)
    dt = time.perf_counter() - t0
    n = int(max(64, min(w.M, 64 * target_s / max(dt, 1e-6))))
    rows = datagen.sample_rows(1, w.M, n)
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=rows, lib=lib)
    dt = time.perf_counter() - t0
    flops = 2.0 * len(rows) * w.N * w.K
    wv = datagen.WORKLOADS[3]
    x, W = datagen.gemv_inputs(wv)
    t0 = time.perf_counter()
    oracle.gemv(x, W, lib=lib)
    dtv = time.perf_counter() - t0
    # one core: the whole 256^3 GEMM and the whole GEMV
    w0 = datagen.WORKLOADS[0]
    A0, B0 = datagen.gemm_inputs(w0)
    t0 = time.perf_counter()
    oracle.gemm(A0, B0, nthreads=1, lib=lib)
    dt0 = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gemv(x, W, nthreads=1, lib=lib)
    dtv1 = time.perf_counter() - t0
    from gemv_tile_pipelined_amd import metrics

    return {
        "value": flops / dt / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"gemm 4096^3 on {len(rows)} of 4096 seeded output rows x 4096 cols x K 4096 "
        f"({flops / 2:.3g} FP64 FMAs, {dt:.1f} s); FP64 triple loop, OpenMP over rows",
        "seconds": dt,
        "gemv_gbps": metrics.gemv_bytes(wv.N, wv.K) / dtv / 1e9,
        "gemv_seconds": dtv,
        "single_core": {
            "gemm_256cube_gflops": 2.0 * w0.M * w0.N * w0.K / dt0 / 1e9,
            "gemm_256cube_seconds": dt0,
            "gemv_gbps": metrics.gemv_bytes(wv.N, wv.K) / dtv1 / 1e9,
            "gemv_seconds": dtv1,
        },
        "cpu_model": _cpu_model(),
    }


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(
            "bench.py measures one GPU only: the library has no multi-GPU path "
            "(the GEMM would shard by output columns with no exchange, the GEMV by rows of W).",
            file=sys.stderr,
        )
        sys.exit(2)

    import numpy as np
    import torch

    import datagen
    import gemv_tile_pipelined_amd as gt
    from gemv_tile_pipelined_amd import metrics

    gt.load_library()  # fails loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    # ---- inputs, resident in HBM before timing --------------------------
    wg = datagen.WORKLOADS[1]
    A0, B0 = datagen.gemm_inputs(wg)
    gemm_sets = []
    for s in range(GEMM_SETS):
        A = torch.from_numpy(A0).to(dev)
        B = torch.from_numpy(B0).to(dev)
        if s:  # distinct data per set (a cheap seeded permutation of rows)
            A = A.roll(s, 0).contiguous()
            B = B.roll(-s, 0).contiguous()
        D = torch.empty((wg.M, wg.N), dtype=torch.float16, device=dev)
        gemm_sets.append((A, B, D))
    wv = datagen.WORKLOADS[3]
    x0, W0 = datagen.gemv_inputs(wv)
    x = torch.from_numpy(x0).to(dev)
    Wt = torch.from_numpy(W0).to(dev)
    gemv_sets = [(Wt if c == 0 else Wt.clone(), torch.empty((wv.N,), dtype=torch.float16, device=dev)) for c in range(GEMV_COPIES)]
    M, N, K = wg.M, wg.N, wg.K
    # The decode batch's activations and the bf16 inputs are resident too,
    # so no host work idles the GPU between the timed sections.
    wd = datagen.DECODE_BATCH
    Ad0, _ = datagen.gemm_inputs(wd)
    Ad = torch.from_numpy(Ad0).to(dev)
    Dd = [torch.empty((wd.M, wd.N), dtype=torch.float16, device=dev) for _ in range(GEMV_COPIES)]

    # numpy has no bfloat16: datagen returns bf16 bit patterns, viewed as such.
    def bf16_tensor(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    Ab0, Bb0 = datagen.gemm_inputs(wg, bf16=True)
    Ab, Bb = bf16_tensor(Ab0), bf16_tensor(Bb0)
    Db = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    xb0, Wb0 = datagen.gemv_inputs(wv, bf16=True)
    xb, Wb = bf16_tensor(xb0), bf16_tensor(Wb0)
    gemv_b = [(Wb if c == 0 else Wb.clone(), torch.empty((wv.N,), dtype=torch.bfloat16, device=dev)) for c in range(GEMV_COPIES)]
    torch.cuda.synchronize(dev)

    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream

    def step(i, ev=None):
        A, B, D = gemm_sets[i % GEMM_SETS]
        if ev:
            ev[0].record(stream)
        st = gt.gemm_f16_ptr(A.data_ptr(), B.data_ptr(), D.data_ptr(), M, N, K, sh)
        if ev:
            ev[1].record(stream)
        for W, y in gemv_sets:
            st |= gt.gemv_f16_ptr(x.data_ptr(), W.data_ptr(), y.data_ptr(), wv.N, wv.K, sh)
        if ev:
            ev[2].record(stream)
        if st:
            raise RuntimeError(f"library call failed: {gt.status_string(st)}")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize(dev)

    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, events[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0

    gemm_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
    gemv_ms = np.array([e[1].elapsed_time(e[2]) for e in events])

    def us_stats(ms, per=1):
        us = np.asarray(ms) * 1e3 / per
        return {"mean": round(float(us.mean()), 2), "median": round(float(np.median(us)), 2),
                "min": round(float(us.min()), 2), "p90": round(float(np.percentile(us, 90)), 2)}
    gemm_s = float(gemm_ms.mean()) / 1e3
    gemv_s = float(gemv_ms.mean()) / 1e3 / GEMV_COPIES
    flops = metrics.gemm_flops(M, N, K)
    gemm_tflops = flops / gemm_s / 1e12
    gemv_bytes = metrics.gemv_bytes(wv.N, wv.K)
    gemv_gbps = gemv_bytes / gemv_s / 1e9

    # ---- decode batch (8 activation rows against the GEMV's weight shape) --
    # Timed on its own after the steps: 5 launches per event pair, one per W
    # copy, so every launch streams its B from HBM.

    def decode_batch():
        st = 0
        for c, (W, _) in enumerate(gemv_sets):
            st |= gt.gemm_f16_ptr(Ad.data_ptr(), W.data_ptr(), Dd[c].data_ptr(), wd.M, wd.N, wd.K, sh)
        if st:
            raise RuntimeError(f"library call failed: {gt.status_string(st)}")

    for _ in range(SECTION_WARMUP):
        decode_batch()
    dev_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(DECODE_REPS)]
    torch.cuda.synchronize(dev)
    for e in dev_events:
        e[0].record(stream)
        decode_batch()
        e[1].record(stream)
    torch.cuda.synchronize(dev)
    decode_s = float(np.mean([e[0].elapsed_time(e[1]) for e in dev_events])) / 1e3 / GEMV_COPIES
    decode_bytes = metrics.gemm_bytes(wd.M, wd.N, wd.K)
    decode_gbps = decode_bytes / decode_s / 1e9

    # ---- bf16: the same GEMM and GEMV shapes on bf16 inputs -----------------

    def bf16_step(ev=None):
        if ev:
            ev[0].record(stream)
        st = gt.gemm_bf16_ptr(Ab.data_ptr(), Bb.data_ptr(), Db.data_ptr(), M, N, K, sh)
        if ev:
            ev[1].record(stream)
        for W, y in gemv_b:
            st |= gt.gemv_bf16_ptr(xb.data_ptr(), W.data_ptr(), y.data_ptr(), wv.N, wv.K, sh)
        if ev:
            ev[2].record(stream)
        if st:
            raise RuntimeError(f"library call failed: {gt.status_string(st)}")

    for _ in range(SECTION_WARMUP):
        bf16_step()
    bf_events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(BF16_REPS)]
    torch.cuda.synchronize(dev)
    for e in bf_events:
        bf16_step(e)
    torch.cuda.synchronize(dev)
    gemm_bf16_s = float(np.mean([e[0].elapsed_time(e[1]) for e in bf_events])) / 1e3
    gemv_bf16_s = float(np.mean([e[1].elapsed_time(e[2]) for e in bf_events])) / 1e3 / GEMV_COPIES
    gemm_bf16_tflops = flops / gemm_bf16_s / 1e12
    gemv_bf16_gbps = gemv_bytes / gemv_bf16_s / 1e9
    del gemv_b, Wb, Ab, Bb, Db

    # ---- the vendor BLAS on the same inputs, same process (reference) ----
    # The part's power-limited clock differs from box to box by several per
    # cent; the vendor GEMM timed here, after the steps, shows where a box
    # stands.  Not part of the timed region, nor of `value`.
    vendor_events = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(VENDOR_REPS)]
    for i in range(SECTION_WARMUP):
        A, B, D = gemm_sets[i % GEMM_SETS]
        torch.matmul(A, B.t(), out=D)
    torch.cuda.synchronize(dev)
    for i, e in enumerate(vendor_events):
        A, B, D = gemm_sets[i % GEMM_SETS]
        e[0].record(stream)
        torch.matmul(A, B.t(), out=D)
        e[1].record(stream)
    torch.cuda.synchronize(dev)
    vendor_gemm_s = float(np.mean([e[0].elapsed_time(e[1]) for e in vendor_events])) / 1e3

    # The part's own compute peak, for context next to the published one the
    # rooflines use: dense fp16 MFMA = CUs x 4096 flop per clock at the peak
    # engine clock (the published 2.5 PFLOP/s is 256 CUs x 4096 x 2.4 GHz).
    # The memory clock the runtime reports does not give the HBM3E data rate
    # (2 GHz x 8192 bits x 2 is half of it), so HBM uses the published peak.
    caps = gt.device_caps()
    device = {
        **caps,
        "fp16_mfma_peak_from_clock_tflops": round(caps["num_cus"] * 4096 * caps["clock_khz"] * 1e3 / 1e12, 1),
        "peaks_used": "published: 2500 TFLOP/s dense fp16/bf16, 8000 GB/s HBM",
    }

    cpu = cpu_baseline(args.cpu_seconds)

    def traffic(kind):
        # HBM-side bytes per launch, or None once the kernels have changed
        # since the counters were taken.
        if kernel_sources_sha256() != MEASURED_TRAFFIC["sources_sha256"]:
            return None
        t = MEASURED_TRAFFIC[kind]
        return int((t["fetch_kib"] + t["write_kib"]) * 1024)

    line = {
        "metric": METRIC,
        "value": round(gemm_tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {
            "workload": "gemm_f16 D=A·Bᵀ 4096x4096x4096 + 5x gemv_f16 y=x·Wᵀ 4096x14336 (5 distinct W), "
            "fp16 in/out, fp32 accumulate",
            "M": M,
            "N": N,
            "K": K,
            "gemv_N": wv.N,
            "gemv_K": wv.K,
            "parallelism": "single GPU",
        },
        "roofline": {
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": metrics.PEAK_FP16_MFMA_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / metrics.PEAK_FP16_MFMA_TFLOPS, 4),
            "traffic": traffic("gemm"),
            "kernel": "gemm_kernel",
            "us_per_launch": round(gemm_s * 1e6, 2),
            "us_stats": us_stats(gemm_ms),
        },
        "gemv": {
            "value": round(gemv_gbps, 1),
            "unit": "GB/s",
            "us_per_launch": round(gemv_s * 1e6, 2),
            "us_stats": us_stats(gemv_ms, GEMV_COPIES),
            "roofline": {
                "bound": "hbm",
                "achieved": round(gemv_gbps, 1),
                "peak": metrics.PEAK_HBM_GBPS,
                "unit": "GB/s",
                "frac": round(gemv_gbps / metrics.PEAK_HBM_GBPS, 4),
                "traffic": traffic("gemv"),
                "kernel": "gemv_kernel",
            },
        },
        "decode_batch": {
            "workload": f"gemm_f16 D=A·Bᵀ {wd.M}x{wd.N}x{wd.K} (5 distinct B), skinny path",
            "value": round(decode_gbps, 1),
            "unit": "GB/s",
            "us_per_launch": round(decode_s * 1e6, 2),
            "tflops": round(metrics.gemm_flops(wd.M, wd.N, wd.K) / decode_s / 1e12, 2),
            "roofline": {
                "bound": "hbm",
                "achieved": round(decode_gbps, 1),
                "peak": metrics.PEAK_HBM_GBPS,
                "unit": "GB/s",
                "frac": round(decode_gbps / metrics.PEAK_HBM_GBPS, 4),
                "traffic": traffic("decode"),
                "kernel": "gemm_skinny_lds_kernel",
            },
        },
        "bf16": {
            "workload": f"gemm_bf16 {M}x{N}x{K} and gemv_bf16 {wv.N}x{wv.K} (5 distinct W), "
            "bf16 in/out, fp32 accumulate",
            "gemm_tflops": round(gemm_bf16_tflops, 2),
            "gemm_us_per_launch": round(gemm_bf16_s * 1e6, 2),
            "gemm_frac": round(gemm_bf16_tflops / metrics.PEAK_BF16_MFMA_TFLOPS, 4),
            "gemm_peak": metrics.PEAK_BF16_MFMA_TFLOPS,
            "gemv_gbps": round(gemv_bf16_gbps, 1),
            "gemv_us_per_launch": round(gemv_bf16_s * 1e6, 2),
            "gemv_frac": round(gemv_bf16_gbps / metrics.PEAK_HBM_GBPS, 4),
            "gemm_traffic": traffic("gemm_bf16"),
            "gemv_traffic": traffic("gemv_bf16"),
        },
        "vendor_same_box": {
            "kind": "torch.matmul (vendor BLAS) on the same fp16 4096^3 inputs, timed after the steps",
            "gemm_us_per_launch": round(vendor_gemm_s * 1e6, 2),
            "gemm_tflops": round(flops / vendor_gemm_s / 1e12, 2),
            "ours_over_vendor_time": round(gemm_s / vendor_gemm_s, 4),
        },
        "device": device,
        "cpu_baseline": cpu,
        "context": "pages' figures (other hardware, BF16 GEMM): 36.13 TFLOP/s at 4096^3 on an SM120 GeForce; "
        "GEMV 695 GB/s (torch.compile) and 708 GB/s (best TileLang) on an RTX A6000",
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
