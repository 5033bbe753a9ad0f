"""Benchmark of the FP16 GEMM / GEMV hot path on one MI355X.

One step = one gemm_f16 at M = N = K = 4096 plus five gemv_f16 at N = 4096,
K = 14336, one over each of five distinct copies of W (the whole hot path;
587 MB of W per step, more than twice the 256 MB MALL, so every GEMV streams
its W from HBM rather than from cache), on seeded synthetic fp16 inputs
already resident in device memory.  The GEMM rotates over 3 input sets.

Before the W warm-up steps the steps run for --settle-s seconds (default
0.5 s): under sustained load the part's power-managed clocks take a few
tenths of a second to settle, and without this the first timed steps run on
a clock that the kernels never see in steady use.  Both phases are untimed.

Prints ONE JSON line on stdout:
  value        GEMM TFLOP/s (2·M·N·K / mean GEMM kernel time, HIP events on
               the stream the kernels run on, created without the
               system-scope fence: see TimingEvent)
  roofline     GEMM against the dense fp16 MFMA peak
  gemv         GEMV GB/s (algorithmic bytes 2·(N·K + K + N) / mean kernel time,
               the five back-to-back launches of a step timed together)
               with its own roofline against the HBM peak
  configs      the other workloads, each timed on its own after the steps with
               its own roofline: GEMM 256^3 (latency-bound; a correctness
               size), GEMM 4000x4032x4104 (ragged edges) and GEMM 8192^3
  vendor_same_box  torch.matmul (the vendor BLAS) and gemm_f16 on the same
               4096^3 input sets, timed interleaved call by call after the
               steps, so both see one clock state
  decode_batch the 8x4096x14336 GEMM (skinny path) in GB/s, timed on its own
  bf16         gemm_bf16 at 4096^3 and gemv_bf16 at 4096x14336
  clock        the clock the MFMAs run at, from per-workgroup timestamps of the
               GEMM kernel (gemvtile_gemm_f16_timed) while 4096^3 launches run
               back to back on the uniform inputs and then on all-zero inputs,
               with the time split into prologue + K loop, epilogue and the
               spread of workgroup end times, and socket power (amdsmi,
               read-only) alongside: the part's power limit sets the clock
  cpu_baseline the CPU oracle (FP64, OpenMP) on a bounded sample of the same
               workloads: the 4096^3 GEMM (rows sized to the time budget), the
               ragged GEMM in full, the 8192^3 GEMM on its 64 seeded rows and
               the GEMV in full
Usage: python bench.py [--gpus 1] [--steps 100] [--warmup 2000] [--settle-s 0.5]
                       [--only gemm|gemv|decode|bf16|configs|vendor|clock|copy|gemm_variants|gemv_variants]
--only runs the steps (or, for decode/bf16/configs/vendor/clock, that
section alone after the same settle phase) and prints the line without the
other sections; it exists so that profiler runs time one kernel family at a
time.  --only copy runs nothing of the library: 20 device-to-device copies of
a 256 MiB buffer, the known-size reference that hardware traffic counters
are calibrated against.  --only gemm_variants / gemv_variants time the
internal ablation variants (gemvtile_gemm_f16_variant / _gemv_f16_variant)
against each other after 1 s of the same rotation untimed: in each round,
each variant in turn runs one untimed launch (which absorbs the switch from
the previous variant) and then a timed block between two events, of four
launches (GEMM) or of five launches over five copies of W (GEMV); one line
per variant and shape.  Before each GEMV block a 512 MiB buffer is read
(untimed), so no variant finds copies of W left in the 256 MB last-level
cache.
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
GEMM_SETS = 3
GEMV_COPIES = 5
DECODE_REPS = 20  # event pairs around 5 decode-batch launches
BF16_REPS = 50  # event triples around one gemm_bf16 and 5 gemv_bf16
SECTION_SETTLE_S = 0.25  # seconds of untimed calls before each section after the steps
VENDOR_REPS = 50  # interleaved pairs (ours, vendor) of timed 4096^3 GEMMs
CONFIG_REPS = {0: 200, 2: 50, 4: 10}  # timed launches per extra workload
# Beyond-L2 traffic per launch measured with rocprofv3 --pmc FETCH_SIZE and
# WRITE_SIZE (KiB per dispatch, each scaled by what the same counter reads for
# a device copy of known size: x2.000 for FETCH_SIZE, x1.000 for WRITE_SIZE),
# valid only for the kernel sources whose SHA-256 is recorded here; the
# summary and commands are in profiles/traffic_fetch_write_size.md.
MEASURED_TRAFFIC = {
    "sources_sha256": "7ad5b1342ccb7e4ffd74183bf3e069855fa50d3069fc765de71172d24c3f256a",
    "gemm": {"fetch_kib": 98443.0 * 2.0, "write_kib": 32791.6 * 1.0},
    "gemv": {"fetch_kib": 57482.6 * 2.0, "write_kib": 64.0 * 1.0},
    "decode": {"fetch_kib": 58267.0 * 2.0, "write_kib": 64.0 * 1.0},
    "gemm_bf16": {"fetch_kib": 98442.0 * 2.0, "write_kib": 32793.2 * 1.0},
    "gemv_bf16": {"fetch_kib": 57482.5 * 2.0, "write_kib": 64.0 * 1.0},
}
KERNEL_SOURCES = ("device_common.hpp", "gemm.hip", "gemm_kernel.hpp", "gemm_plain.hip", "gemv.hip", "kernels.hpp",
                  "ring.hpp", "skinny.hip", "tile_order.hpp")


def kernel_sources_sha256() -> str:
    import hashlib

    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "gemv_tile_pipelined_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


_HIP = None
HIP_EVENT_DISABLE_SYSTEM_FENCE = 0x20000000


_FENCED_EVENTS = False


def new_event():
    """A timing event: fence-free (TimingEvent), or torch's default one with
    --fenced-events."""
    if _FENCED_EVENTS:
        import torch

        return torch.cuda.Event(enable_timing=True)
    return TimingEvent()


class TimingEvent:
    """A HIP event for timing only (record on a stream, elapsed time between
    two), created with hipEventDisableSystemFence.  A default event makes a
    system-scope release when it is recorded: an L2 write-back and invalidate
    that lands inside the timed interval and leaves the next kernel to start
    on an invalidated L2.  Timing events need neither (the elapsed time is
    read after a device synchronisation), and without them a per-launch
    event pair measures the kernel rather than the fence.  Same interface as
    torch.cuda.Event(enable_timing=True) for record() and elapsed_time();
    the HIP runtime is the one torch has loaded."""

    def __init__(self):
        import ctypes

        global _HIP
        if _HIP is None:
            path = next((ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln), None)
            if path is None:
                raise RuntimeError("the HIP runtime is not loaded (torch.cuda must be initialised first)")
            _HIP = ctypes.CDLL(path)
            _HIP.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            _HIP.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            _HIP.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
            _HIP.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self._ct = ctypes
        self.ev = ctypes.c_void_p()
        st = _HIP.hipEventCreateWithFlags(ctypes.byref(self.ev), HIP_EVENT_DISABLE_SYSTEM_FENCE)
        if st:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")

    def record(self, stream):
        st = _HIP.hipEventRecord(self.ev, self._ct.c_void_p(stream.cuda_stream))
        if st:
            raise RuntimeError(f"hipEventRecord failed ({st})")

    def elapsed_time(self, end) -> float:
        """Milliseconds from this event to `end` (both must have completed)."""
        ms = self._ct.c_float()
        st = _HIP.hipEventElapsedTime(self._ct.byref(ms), self.ev, end.ev)
        if st:
            raise RuntimeError(f"hipEventElapsedTime failed ({st})")
        return ms.value

    def __del__(self):
        if _HIP is not None and self.ev:
            _HIP.hipEventDestroy(self.ev)


def parse():
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=100)
    p.add_argument("--warmup", type=int, default=2000)
    p.add_argument("--settle-s", type=float, default=0.5, help="seconds of untimed steps before the warm-up steps")
    p.add_argument("--cpu-seconds", type=float, default=8.0, help="target CPU time of the 4096^3 oracle sample")
    p.add_argument("--only", choices=("gemm", "gemv", "decode", "bf16", "configs", "vendor", "clock", "copy",
                                      "gemm_variants", "gemv_variants"), default=None)
    p.add_argument("--variants", default="0", help="--only gemm_variants / gemv_variants: variant numbers, "
                   "comma-separated (gemm: -1 = the vendor GEMM, torch.matmul; -2 = gemm_splitk_f16 with a workspace; "
                   "-3 = gemm_bias_f16 with a bias and ReLU; -4 = gemm_bf16 on the same shapes)")
    p.add_argument("--shapes", default="4096x4096x4096", help="--only gemm_variants: MxNxK list; gemv_variants: NxK "
                   "list, or RxNxK for gemm_f16 variants on an R-row activation batch against W [N,K]")
    p.add_argument("--data", choices=("uniform", "zero", "mant7"), default="uniform",
                   help="--only gemm_variants inputs: seeded U(-1,1) fp16, all zeros, or the same U(-1,1) fp16 values "
                   "with the low 3 of their 10 mantissa bits cleared (the mantissa width of bf16)")
    p.add_argument("--reps", type=int, default=24, help="--only gemm_variants / gemv_variants timed rounds")
    p.add_argument("--clock-s", type=float, default=2.0, help="seconds of sampled load per data set in the clock section")
    p.add_argument("--fenced-events", action="store_true", help="time with default HIP events (torch.cuda.Event), "
                   "which make a system-scope release when recorded, instead of fence-free ones (for comparison)")
    return p.parse_args()


def cpu_baseline(target_s: float):
    """The oracle as it stands, on the workloads the GPU runs (bounded)."""
    import numpy as np

    import datagen
    import oracle
    from gemv_tile_pipelined_amd import metrics

    lib = oracle.load()
    threads = oracle.max_threads(lib)
    out = {}
    # 4096^3: calibrate on 256 rows (16 per thread on a 16-core share, so
    # the threads are evenly loaded), then as many rows as fit the budget:
    # the whole GEMM when it fits
    w = datagen.WORKLOADS[1]
    A, B = datagen.gemm_inputs(w)
    rows = datagen.sample_rows(1, w.M, 256)
    oracle.gemm(A, B, rows=rows[:16], lib=lib)
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=rows, lib=lib)
    dt = time.perf_counter() - t0
    n = int(max(256, min(w.M, 256 * target_s / max(dt, 1e-6))))
    rows = datagen.sample_rows(1, w.M, n) if n < w.M else np.arange(w.M)
    t0 = time.perf_counter()
    oracle.gemm(A, B, rows=None if n >= w.M else rows, lib=lib)
    dt1 = time.perf_counter() - t0
    flops1 = 2.0 * len(rows) * w.N * w.K
    del A, B
    # the ragged GEMM in full
    w2 = datagen.WORKLOADS[2]
    A2, B2 = datagen.gemm_inputs(w2)
    t0 = time.perf_counter()
    oracle.gemm(A2, B2, lib=lib)
    dt2 = time.perf_counter() - t0
    del A2, B2
    # 8192^3 on its 64 seeded rows
    w4 = datagen.WORKLOADS[4]
    A4, B4 = datagen.gemm_inputs(w4)
    rows4 = datagen.sample_rows(4, w4.M, 64)
    t0 = time.perf_counter()
    oracle.gemm(A4, B4, rows=rows4, lib=lib)
    dt4 = time.perf_counter() - t0
    del A4, B4
    # the GEMV in full, all cores and one core
    wv = datagen.WORKLOADS[3]
    x, W = datagen.gemv_inputs(wv)
    t0 = time.perf_counter()
    oracle.gemv(x, W, lib=lib)
    dtv = time.perf_counter() - t0
    t0 = time.perf_counter()
    oracle.gemv(x, W, nthreads=1, lib=lib)
    dtv1 = time.perf_counter() - t0
    # one core: the whole 256^3 GEMM
    w0 = datagen.WORKLOADS[0]
    A0, B0 = datagen.gemm_inputs(w0)
    t0 = time.perf_counter()
    oracle.gemm(A0, B0, nthreads=1, lib=lib)
    dt0 = time.perf_counter() - t0
    out = {
        "value": flops1 / dt1 / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"gemm 4096^3 in full ({flops1 / 2:.3g} FP64 FMAs, {dt1:.2f} s)" if len(rows) == w.M else
                   f"gemm 4096^3 on {len(rows)} of 4096 seeded output rows x 4096 cols x K 4096 "
                   f"({flops1 / 2:.3g} FP64 FMAs, {dt1:.2f} s)") + "; FP64 triple loop, OpenMP over rows",
        "seconds": dt1,
        "ragged_4000x4032x4104_full": {"seconds": dt2, "tflops": metrics.gemm_flops(w2.M, w2.N, w2.K) / dt2 / 1e12},
        "gemm_8192_64_rows": {"seconds": dt4, "tflops": 2.0 * len(rows4) * w4.N * w4.K / dt4 / 1e12},
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
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class ClockSampler:
    """Samples the GPU's engine clocks and socket power through amdsmi (the
    ROCm system-management library; read-only queries) in a background
    thread."""

    def __init__(self, device_index=0, period_s=0.005):
        import threading

        import amdsmi

        self.amdsmi = amdsmi
        amdsmi.amdsmi_init(amdsmi.AmdSmiInitFlags.INIT_AMD_GPUS)
        self.handle = amdsmi.amdsmi_get_processor_handles()[device_index]
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def read(self):
        m = self.amdsmi.amdsmi_get_gpu_metrics_info(self.handle)
        clks = [c for c in (m.get("current_gfxclks") or []) if isinstance(c, (int, float)) and 0 < c < 10000]
        one = m.get("current_gfxclk")
        if not clks and isinstance(one, (int, float)) and 0 < one < 10000:
            clks = [one]
        power = m.get("current_socket_power")
        if not isinstance(power, (int, float)) or power <= 0 or power > 100000:
            power = m.get("average_socket_power")
        return {"clks": clks, "power": power if isinstance(power, (int, float)) and 0 < power < 100000 else None}

    def _run(self):
        import time as _t

        while not self._stop.is_set():
            try:
                self.samples.append(self.read())
            except Exception as e:  # a failing query ends the sampling, not the bench
                self.samples.append({"error": repr(e)})
                return
            _t.sleep(self.period)

    def start(self):
        self._thread.start()

    def stop(self):
        self._stop.set()
        self._thread.join()
        return self.samples

    def power_cap_w(self):
        try:
            info = self.amdsmi.amdsmi_get_power_cap_info(self.handle)
            cap = info.get("power_cap")
            return cap / 1e6 if isinstance(cap, (int, float)) and cap > 1e5 else cap
        except Exception:
            return None

    def close(self):
        try:
            self.amdsmi.amdsmi_shut_down()
        except Exception:
            pass


def summarize_clock(samples):
    import numpy as np

    good = [x for x in samples if "clks" in x and x["clks"]]
    if not good:
        return {"samples": len(samples), "error": next((x["error"] for x in samples if "error" in x), "no clock data")}
    # drop the first tenth (the load ramping up)
    good = good[len(good) // 10:]
    per_xcd = np.array([x["clks"] for x in good if len(x["clks"]) == len(good[0]["clks"])], dtype=float)
    mean_clk = per_xcd.mean(axis=1)
    pw = np.array([x["power"] for x in good if x["power"] is not None], dtype=float)
    out = {
        "samples": len(good),
        "gfxclk_mhz_mean": round(float(mean_clk.mean()), 1),
        "gfxclk_mhz_min": round(float(mean_clk.min()), 1),
        "gfxclk_mhz_max": round(float(mean_clk.max()), 1),
        "per_xcd_mhz_mean": [round(float(v), 1) for v in per_xcd.mean(axis=0)],
    }
    if pw.size:
        out["socket_power_w_mean"] = round(float(pw.mean()), 1)
        out["socket_power_w_max"] = round(float(pw.max()), 1)
    return out


def us_stats(ms, per=1):
    import numpy as np

    us = np.asarray(ms) * 1e3 / per
    return {"mean": round(float(us.mean()), 2), "median": round(float(np.median(us)), 2),
            "min": round(float(us.min()), 2), "p90": round(float(np.percentile(us, 90)), 2)}


def roofline(bound, achieved, peak, unit, traffic=None, kernel=None, **extra):
    r = {"bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic}
    if kernel:
        r["kernel"] = kernel
    r.update(extra)
    return r


def variant_sweep(args, torch, np, gt, datagen, dev):
    """Interleaved timing of ablation variants (see the module doc)."""
    lib = gt.load_library()
    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    variants = [int(v) for v in args.variants.split(",")]
    out = {"only": args.only, "data": args.data, "results": []}

    # a 512 MiB buffer read (not written: no write-backs left behind) before
    # each GEMV variant's block, so none finds W left in the last-level cache
    flush = torch.ones((128 << 20,), dtype=torch.int32, device=dev) if args.only == "gemv_variants" else None
    block = 4 if args.only == "gemm_variants" else 1

    def interleaved(run, n_per):
        t_end = time.perf_counter() + 1.0
        i = 0
        while time.perf_counter() < t_end:
            for v in variants:
                run(v, i)
            i += 1
            torch.cuda.synchronize(dev)
        ev = {v: [] for v in variants}
        for r in range(args.reps):
            for v in variants:
                if flush is not None:
                    flush.max()
                run(v, r)  # untimed: absorbs the switch from the previous variant
                e0, e1 = new_event(), new_event()
                e0.record(stream)
                for b in range(block):
                    run(v, r + 1 + b)
                e1.record(stream)
                ev[v].append((e0, e1))
        torch.cuda.synchronize(dev)
        return {v: np.array([a.elapsed_time(b) for a, b in ev[v]]) * 1e3 / (n_per * block) for v in variants}

    for shape in args.shapes.split(","):
        dims = [int(t) for t in shape.split("x")]
        if args.only == "gemm_variants":
            M, N, K = dims
            sets = []
            for i in range(3 if M * N * K <= 4096 ** 3 else 1):
                if args.data == "zero":
                    A = torch.zeros((M, K), dtype=torch.float16, device=dev)
                    B = torch.zeros((N, K), dtype=torch.float16, device=dev)
                else:
                    A = torch.from_numpy(datagen.uniform_f16(50 + i, 0, (M, K), -1.0, 1.0)).to(dev)
                    B = torch.from_numpy(datagen.uniform_f16(50 + i, 1, (N, K), -1.0, 1.0)).to(dev)
                    if args.data == "mant7":
                        A.view(torch.int16).bitwise_and_(-8)
                        B.view(torch.int16).bitwise_and_(-8)
                sets.append((A, B, torch.empty((M, N), dtype=torch.float16, device=dev)))
            if -2 in variants:
                ws = gt.alloc_splitk_workspace(sets[0][0], sets[0][1])
            if -3 in variants:
                bias = torch.from_numpy(datagen.uniform_f16(1, 3, (N,), -4.0, 4.0)).to(dev)
            if -4 in variants:
                bsets = [(A.to(torch.bfloat16), B.to(torch.bfloat16), torch.empty((M, N), dtype=torch.bfloat16,
                                                                                   device=dev)) for A, B, _ in sets]

            def run(v, i):
                A, B, D = sets[i % len(sets)]
                if v == -1:
                    torch.matmul(A, B.t(), out=D)
                elif v == -2:
                    gt.gemm_splitk_f16(A, B, D, workspace=ws)
                elif v == -3:
                    gt.gemm_bias_f16(A, B, bias, gt.ACT_RELU, D)
                elif v == -4:
                    Ab, Bb, Db = bsets[i % len(bsets)]
                    gt.gemm_bf16(Ab, Bb, Db)
                else:
                    st = lib.gemvtile_gemm_f16_variant(A.data_ptr(), B.data_ptr(), D.data_ptr(), M, N, K, sh, v)
                    if st:
                        raise RuntimeError(f"variant {v}: {gt.status_string(st)}")

            us = interleaved(run, 1)
            work, unit = 2.0 * M * N * K, "TFLOP/s"
        else:
            rows = dims[0] if len(dims) == 3 else 0
            N, K = dims[-2], dims[-1]
            x = torch.from_numpy(datagen.uniform_f16(3, 0, (max(rows, 1), K) if rows else (K,), -1.0, 1.0)).to(dev)
            W0 = torch.from_numpy(datagen.uniform_f16(3, 1, (N, K), -0.05, 0.05)).to(dev)
            Ws = [W0] + [W0.clone() for _ in range(GEMV_COPIES - 1)]
            ys = [torch.empty((rows, N) if rows else (N,), dtype=torch.float16, device=dev) for _ in Ws]

            def run(v, i):
                for W, y in zip(Ws, ys):
                    if rows:
                        st = lib.gemvtile_gemm_f16_variant(x.data_ptr(), W.data_ptr(), y.data_ptr(), rows, N, K, sh, v)
                    else:
                        st = lib.gemvtile_gemv_f16_variant(x.data_ptr(), W.data_ptr(), y.data_ptr(), N, K, sh, v)
                    if st:
                        raise RuntimeError(f"variant {v}: {gt.status_string(st)}")

            us = interleaved(run, GEMV_COPIES)
            work, unit = 2.0 * (N * K + max(rows, 1) * (K + N)), "GB/s"
        for v in variants:
            u = us[v]
            rate = work / (u.mean() * 1e-6) / (1e12 if unit == "TFLOP/s" else 1e9)
            print(f"{shape} variant {v}: mean {u.mean():.2f} median {np.median(u):.2f} min {u.min():.2f} us, "
                  f"{rate:.0f} {unit}", file=sys.stderr, flush=True)
            out["results"].append({"shape": shape, "variant": v, "us_mean": round(float(u.mean()), 2),
                                   "us_median": round(float(np.median(u)), 2), "us_min": round(float(u.min()), 2),
                                   "rate": round(rate, 1), "unit": unit})
    print(json.dumps(out), flush=True)


def main():
    global _FENCED_EVENTS
    args = parse()
    _FENCED_EVENTS = args.fenced_events
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
    only = args.only
    if only in ("gemm_variants", "gemv_variants"):
        variant_sweep(args, torch, np, gt, datagen, dev)
        return
    if only == "copy":
        nbytes = 256 << 20
        src = torch.ones(nbytes, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(20):
            dst.copy_(src)
        torch.cuda.synchronize(dev)
        print(json.dumps({"metric": METRIC, "value": None, "only": "copy", "copy_bytes": nbytes, "copies": 20}))
        return
    want = (lambda s: only is None or only == s)

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
    gemv_sets = [(Wt if c == 0 else Wt.clone(), torch.empty((wv.N,), dtype=torch.float16, device=dev))
                 for c in range(GEMV_COPIES)]
    M, N, K = wg.M, wg.N, wg.K
    # The later sections' inputs too, so that no host work (uploads) idles
    # the GPU between sections.
    cfg_inputs = {}
    if want("configs"):
        for cid in (0, 2, 4):
            w = datagen.WORKLOADS[cid]
            Ah, Bh = datagen.gemm_inputs(w)
            cfg_inputs[cid] = (torch.from_numpy(Ah).to(dev), torch.from_numpy(Bh).to(dev),
                               torch.empty((w.M, w.N), dtype=torch.float16, device=dev))
            del Ah, Bh
    wd = datagen.DECODE_BATCH
    if want("decode"):
        Ad = torch.from_numpy(datagen.gemm_inputs(wd)[0]).to(dev)
        Dd = [torch.empty((wd.M, wd.N), dtype=torch.float16, device=dev) for _ in range(GEMV_COPIES)]
    if want("bf16"):
        def bf16_tensor(bits):
            return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

        Ab0, Bb0 = datagen.gemm_inputs(wg, bf16=True)
        Ab, Bb = bf16_tensor(Ab0), bf16_tensor(Bb0)
        Db = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        xb0, Wb0 = datagen.gemv_inputs(wv, bf16=True)
        xb, Wb = bf16_tensor(xb0), bf16_tensor(Wb0)
        gemv_b = [(Wb if c == 0 else Wb.clone(), torch.empty((wv.N,), dtype=torch.bfloat16, device=dev))
                  for c in range(GEMV_COPIES)]
        del Ab0, Bb0, xb0, Wb0
    torch.cuda.synchronize(dev)

    stream = torch.cuda.current_stream(dev)
    sh = stream.cuda_stream
    gemm_on = only in (None, "gemm", "gemv")
    gemv_on = only in (None, "gemm", "gemv")
    if only == "gemm":
        gemv_on = False
    if only == "gemv":
        gemm_on = False

    def check(st):
        if st:
            raise RuntimeError(f"library call failed: {gt.status_string(st)}")

    def step(i, ev=None):
        if ev:
            ev[0].record(stream)
        if gemm_on:
            A, B, D = gemm_sets[i % GEMM_SETS]
            check(gt.gemm_f16_ptr(A.data_ptr(), B.data_ptr(), D.data_ptr(), M, N, K, sh))
        if ev:
            ev[1].record(stream)
        if gemv_on:
            for W, y in gemv_sets:
                check(gt.gemv_f16_ptr(x.data_ptr(), W.data_ptr(), y.data_ptr(), wv.N, wv.K, sh))
        if ev:
            ev[2].record(stream)

    def settle(fn):
        # untimed load until the clocks have settled (see the module doc)
        t_end = time.perf_counter() + args.settle_s
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(20):
                fn(i)
                i += 1
            torch.cuda.synchronize(dev)
        return i

    main_steps = gemm_on or gemv_on
    settled = 0
    if main_steps:
        settled = settle(step)
        for i in range(args.warmup):
            step(i)
    else:
        settled = settle(lambda i: check(gt.gemm_f16_ptr(gemm_sets[i % GEMM_SETS][0].data_ptr(),
                                                          gemm_sets[i % GEMM_SETS][1].data_ptr(),
                                                          gemm_sets[i % GEMM_SETS][2].data_ptr(), M, N, K, sh)))
    torch.cuda.synchronize(dev)

    events = [[new_event() for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    if main_steps:
        for i in range(args.steps):
            step(i, events[i])
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - t0

    flops = metrics.gemm_flops(M, N, K)
    gemv_bytes = metrics.gemv_bytes(wv.N, wv.K)
    line = {
        "metric": METRIC,
        "value": None,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "settle_s": args.settle_s,
        "settle_steps": settled,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "timing_events": "default (system-scope fence)" if _FENCED_EVENTS else "fence-free (hipEventDisableSystemFence)",
        "config": {
            "workload": "gemm_f16 D=A·Bᵀ 4096x4096x4096 + 5x gemv_f16 y=x·Wᵀ 4096x14336 (5 distinct W), "
            "fp16 in/out, fp32 accumulate",
            "M": M, "N": N, "K": K, "gemv_N": wv.N, "gemv_K": wv.K,
            "parallelism": "single GPU",
        },
    }
    if only:
        line["only"] = only

    def traffic(kind):
        # HBM-side bytes per launch, or None once the kernels have changed
        # since the counters were taken.
        if kernel_sources_sha256() != MEASURED_TRAFFIC["sources_sha256"] or kind not in MEASURED_TRAFFIC:
            return None
        t = MEASURED_TRAFFIC[kind]
        return int((t["fetch_kib"] + t["write_kib"]) * 1024)

    if gemm_on and main_steps:
        gemm_ms = np.array([e[0].elapsed_time(e[1]) for e in events])
        gemm_s = float(gemm_ms.mean()) / 1e3
        gemm_tflops = flops / gemm_s / 1e12
        line["value"] = round(gemm_tflops, 2)
        line["roofline"] = roofline("mfma", gemm_tflops, metrics.PEAK_FP16_MFMA_TFLOPS, "TFLOP/s", traffic("gemm"),
                                    "gemm_kernel", us_per_launch=round(gemm_s * 1e6, 2), us_stats=us_stats(gemm_ms))
    if gemv_on and main_steps:
        gemv_ms = np.array([e[1].elapsed_time(e[2]) for e in events])
        gemv_s = float(gemv_ms.mean()) / 1e3 / GEMV_COPIES
        gemv_gbps = gemv_bytes / gemv_s / 1e9
        line["gemv"] = {
            "value": round(gemv_gbps, 1), "unit": "GB/s", "us_per_launch": round(gemv_s * 1e6, 2),
            "us_stats": us_stats(gemv_ms, GEMV_COPIES),
            "roofline": roofline("hbm", gemv_gbps, metrics.PEAK_HBM_GBPS, "GB/s", traffic("gemv"), "gemv_kernel"),
        }
        if only == "gemv":
            line["value"] = None

    def section_settle(fn):
        # untimed calls for SECTION_SETTLE_S seconds before a section's timed
        # calls: a section that changes the load (its own shape, or the
        # vendor's kernel) moves the power-managed clock, which takes a few
        # tenths of a second to settle again
        t_end = time.perf_counter() + SECTION_SETTLE_S
        i = 0
        while time.perf_counter() < t_end:
            for _ in range(4):
                fn(i)
                i += 1
            torch.cuda.synchronize(dev)

    def timed(fn, reps):
        section_settle(fn)
        evs = [[new_event() for _ in range(2)] for _ in range(reps)]
        torch.cuda.synchronize(dev)
        for i, e in enumerate(evs):
            e[0].record(stream)
            fn(i)
            e[1].record(stream)
        torch.cuda.synchronize(dev)
        return np.array([e[0].elapsed_time(e[1]) for e in evs])

    # ---- the other workloads, each with its own roofline -----------------
    if want("configs"):
        cfg_out = {}
        for cid in (0, 2, 4):
            w = datagen.WORKLOADS[cid]
            Ac, Bc, Dc = cfg_inputs[cid]

            def one(i, Ac=Ac, Bc=Bc, Dc=Dc, w=w):
                check(gt.gemm_f16_ptr(Ac.data_ptr(), Bc.data_ptr(), Dc.data_ptr(), w.M, w.N, w.K, sh))

            reps = CONFIG_REPS[cid]
            ms = timed(one, reps)
            s = float(ms.mean()) / 1e3
            tf = metrics.gemm_flops(w.M, w.N, w.K) / s / 1e12
            bound = "latency" if cid == 0 else "mfma"
            cfg_out[w.name] = {
                "M": w.M, "N": w.N, "K": w.K, "us_per_launch": round(s * 1e6, 2), "us_stats": us_stats(ms),
                "tflops": round(tf, 2),
                "roofline": roofline("mfma", tf, metrics.PEAK_FP16_MFMA_TFLOPS, "TFLOP/s", None, "gemm_kernel",
                                     regime=bound),
            }
            del Ac, Bc, Dc
        cfg_inputs.clear()
        line["configs"] = cfg_out

    # ---- our GEMM and the vendor's, interleaved on the same inputs -------
    if want("vendor"):
        def pair(i, ev=None):
            A, B, D = gemm_sets[i % GEMM_SETS]
            if ev:
                ev[0].record(stream)
            check(gt.gemm_f16_ptr(A.data_ptr(), B.data_ptr(), D.data_ptr(), M, N, K, sh))
            if ev:
                ev[1].record(stream)
            torch.matmul(A, B.t(), out=D)
            if ev:
                ev[2].record(stream)

        section_settle(pair)
        vev = [[new_event() for _ in range(3)] for _ in range(VENDOR_REPS)]
        torch.cuda.synchronize(dev)
        for i, e in enumerate(vev):
            pair(i, e)
        torch.cuda.synchronize(dev)
        ours = np.array([e[0].elapsed_time(e[1]) for e in vev])
        theirs = np.array([e[1].elapsed_time(e[2]) for e in vev])
        line["vendor_same_box"] = {
            "kind": "torch.matmul (vendor BLAS) and gemm_f16 on the same fp16 4096^3 input sets, "
            "one call of each per iteration, after the same warm-up",
            "ours_us_per_launch": round(float(ours.mean()) * 1e3, 2),
            "vendor_us_per_launch": round(float(theirs.mean()) * 1e3, 2),
            "ours_us_stats": us_stats(ours), "vendor_us_stats": us_stats(theirs),
            "vendor_tflops": round(flops / (float(theirs.mean()) / 1e3) / 1e12, 2),
            "ours_over_vendor_time": round(float(ours.mean()) / float(theirs.mean()), 4),
        }

    # ---- decode batch (8 activation rows against the GEMV's weight shape) --
    if want("decode"):
        def decode_batch(i):
            for c, (W, _) in enumerate(gemv_sets):
                check(gt.gemm_f16_ptr(Ad.data_ptr(), W.data_ptr(), Dd[c].data_ptr(), wd.M, wd.N, wd.K, sh))

        ms = timed(decode_batch, DECODE_REPS)
        decode_s = float(ms.mean()) / 1e3 / GEMV_COPIES
        decode_gbps = metrics.gemm_bytes(wd.M, wd.N, wd.K) / decode_s / 1e9
        line["decode_batch"] = {
            "workload": f"gemm_f16 D=A·Bᵀ {wd.M}x{wd.N}x{wd.K} (5 distinct B), skinny path",
            "value": round(decode_gbps, 1), "unit": "GB/s", "us_per_launch": round(decode_s * 1e6, 2),
            "tflops": round(metrics.gemm_flops(wd.M, wd.N, wd.K) / decode_s / 1e12, 2),
            "roofline": roofline("hbm", decode_gbps, metrics.PEAK_HBM_GBPS, "GB/s", traffic("decode"),
                                 "gemm_skinny_lds_kernel"),
        }

    # ---- bf16: the same GEMM and GEMV shapes on bf16 inputs ---------------
    if want("bf16"):
        def bf16_step(ev=None):
            if ev:
                ev[0].record(stream)
            check(gt.gemm_bf16_ptr(Ab.data_ptr(), Bb.data_ptr(), Db.data_ptr(), M, N, K, sh))
            if ev:
                ev[1].record(stream)
            for W, y in gemv_b:
                check(gt.gemv_bf16_ptr(xb.data_ptr(), W.data_ptr(), y.data_ptr(), wv.N, wv.K, sh))
            if ev:
                ev[2].record(stream)

        section_settle(lambda i: bf16_step())
        bf_events = [[new_event() for _ in range(3)] for _ in range(BF16_REPS)]
        torch.cuda.synchronize(dev)
        for e in bf_events:
            bf16_step(e)
        torch.cuda.synchronize(dev)
        gemm_bf16_s = float(np.mean([e[0].elapsed_time(e[1]) for e in bf_events])) / 1e3
        gemv_bf16_s = float(np.mean([e[1].elapsed_time(e[2]) for e in bf_events])) / 1e3 / GEMV_COPIES
        line["bf16"] = {
            "workload": f"gemm_bf16 {M}x{N}x{K} and gemv_bf16 {wv.N}x{wv.K} (5 distinct W), "
            "bf16 in/out, fp32 accumulate",
            "gemm_tflops": round(flops / gemm_bf16_s / 1e12, 2),
            "gemm_us_per_launch": round(gemm_bf16_s * 1e6, 2),
            "gemm_frac": round(flops / gemm_bf16_s / 1e12 / metrics.PEAK_BF16_MFMA_TFLOPS, 4),
            "gemm_peak": metrics.PEAK_BF16_MFMA_TFLOPS,
            "gemv_gbps": round(gemv_bytes / gemv_bf16_s / 1e9, 1),
            "gemv_us_per_launch": round(gemv_bf16_s * 1e6, 2),
            "gemv_frac": round(gemv_bytes / gemv_bf16_s / 1e9 / metrics.PEAK_HBM_GBPS, 4),
            "gemm_traffic": traffic("gemm_bf16"),
            "gemv_traffic": traffic("gemv_bf16"),
        }
        del gemv_b, Wb, Ab, Bb, Db

    # ---- the engine clock under sustained GEMM load ---------------------
    if want("clock"):
        clock = {"method": "gemvtile_gemm_f16_timed (the default 256x256 kernel with per-workgroup start / "
                           "K-loop end / end stamps of the 100 MHz real-time and the shader-cycle counters) run "
                           "back to back; the last 20 launches analysed. Socket power and the SMU's clock "
                           "reading sampled alongside with amdsmi (read-only; its readings refresh slowly)."}
        try:
            lib = gt.load_library()
            zero_A = torch.zeros((M, K), dtype=torch.float16, device=dev)
            zero_B = torch.zeros((N, K), dtype=torch.float16, device=dev)
            zero_D = torch.empty((M, N), dtype=torch.float16, device=dev)
            grid = gt.gemm_grid(M, N, K, gt.device_caps()["num_cus"])
            n_keep = 20
            stamps = torch.zeros((n_keep, grid * 8), dtype=torch.int64, device=dev)
            # MFMA cycles per wave of one 256x256 tile: (128/16)^2 blocks x K/32 steps x 16 cycles
            mfma_cycles = (128 // 16) * (128 // 16) * (K // 32) * 16
            for name, operands in (("uniform", [(A_, B_, D_) for A_, B_, D_ in gemm_sets]),
                                   ("zero", [(zero_A, zero_B, zero_D)])):
                def one(i, operands=operands):
                    A_, B_, D_ = operands[i % len(operands)]
                    check(lib.gemvtile_gemm_f16_timed(A_.data_ptr(), B_.data_ptr(), D_.data_ptr(), M, N, K, sh,
                                                      stamps[i % n_keep].data_ptr(), grid * 8))

                section_settle(one)
                sampler = None
                try:
                    sampler = ClockSampler()
                    sampler.start()
                except Exception as e:
                    clock.setdefault("amdsmi_error", repr(e))
                t_end = time.perf_counter() + args.clock_s
                n = 0
                e0, e1 = new_event(), new_event()
                e0.record(stream)
                while time.perf_counter() < t_end or n < n_keep:
                    for _ in range(50):
                        one(n)
                        n += 1
                    torch.cuda.synchronize(dev)
                e1.record(stream)
                torch.cuda.synchronize(dev)
                us = e0.elapsed_time(e1) * 1e3 / n
                entry = {"launches": n, "us_per_launch": round(us, 2), "tflops": round(flops / (us * 1e-6) / 1e12, 1)}
                if sampler is not None:
                    samples = sampler.stop()
                    entry["amdsmi"] = summarize_clock(samples)
                    cap = sampler.power_cap_w()
                    if cap is not None:
                        clock["power_cap_w"] = cap
                    sampler.close()
                st = stamps.cpu().numpy().reshape(n_keep, grid, 8).astype(np.float64)
                r0, c0, r1, c1, r2, c2 = (st[..., k] for k in range(6))
                xcc = (st[..., 7].astype(np.int64) & 0xF)
                clk_mhz = (c2 - c0) / (r2 - r0) * 100.0  # per workgroup and launch
                span_us = (r2.max(axis=1) - r0.min(axis=1)) / 100.0  # per launch
                loop_us = (r1 - r0) / 100.0
                epi_us = (r2 - r1) / 100.0
                end_spread_us = (r2.max(axis=1) - np.median(r2, axis=1)) / 100.0
                start_spread_us = (r0.max(axis=1) - r0.min(axis=1)) / 100.0
                loop_cycles = c1 - c0
                entry["timed"] = {
                    "clock_mhz_median": round(float(np.median(clk_mhz)), 1),
                    "clock_mhz_p10_p90": [round(float(np.percentile(clk_mhz, 10)), 1),
                                          round(float(np.percentile(clk_mhz, 90)), 1)],
                    "clock_mhz_per_xcd": [round(float(np.median(clk_mhz[xcc == x])), 1) for x in range(8)
                                          if (xcc == x).any()],
                    "launch_span_us_median": round(float(np.median(span_us)), 2),
                    "start_spread_us_median": round(float(np.median(start_spread_us)), 2),
                    "prologue_and_k_loop_us_median": round(float(np.median(loop_us)), 2),
                    "epilogue_us_median": round(float(np.median(epi_us)), 2),
                    "end_spread_us_median": round(float(np.median(end_spread_us)), 2),
                    "k_loop_cycles_median": round(float(np.median(loop_cycles))),
                    "mfma_cycles_per_wave": mfma_cycles,
                    "mfma_busy_in_k_loop": round(mfma_cycles / float(np.median(loop_cycles)), 4),
                }
                mhz = entry["timed"]["clock_mhz_median"]
                entry["mfma_peak_at_this_clock_tflops"] = round(gt.device_caps()["num_cus"] * 4096 * mhz * 1e6 / 1e12, 1)
                entry["frac_of_peak_at_this_clock"] = round(entry["tflops"] / entry["mfma_peak_at_this_clock_tflops"], 4)
                clock[name] = entry
            del zero_A, zero_B, zero_D, stamps
        except Exception as e:  # the clock evidence is optional; the bench line is not
            clock["error"] = repr(e)
        line["clock"] = clock

    # The part's own compute peak, for context next to the published one the
    # rooflines use: dense fp16 MFMA = CUs x 4096 flop per clock at the peak
    # engine clock (the published 2.5 PFLOP/s is 256 CUs x 4096 x 2.4 GHz).
    caps = gt.device_caps()
    line["device"] = {
        **caps,
        "fp16_mfma_peak_from_clock_tflops": round(caps["num_cus"] * 4096 * caps["clock_khz"] * 1e3 / 1e12, 1),
        "peaks_used": "published: 2500 TFLOP/s dense fp16/bf16, 8000 GB/s HBM",
    }
    if only is None:
        line["cpu_baseline"] = cpu_baseline(args.cpu_seconds)
        line["context"] = ("pages' figures (other hardware, BF16 GEMM): 36.13 TFLOP/s at 4096^3 on an SM120 "
                           "GeForce; GEMV 695 GB/s (torch.compile) and 708 GB/s (best TileLang) on an RTX A6000")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
