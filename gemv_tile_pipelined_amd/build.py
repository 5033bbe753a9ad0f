"""Build the gfx950 library libgemvtile.so in-tree with hipcc.

Usage: python -m gemv_tile_pipelined_amd.build   (or call build_library()).
The library is compiled for gfx950 only.  Packed-FP32 instructions are
disabled for the device code (-packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.

The GEMM kernels issue their 16x16x32 MFMAs as inline asm with the
accumulators bound to AGPRs.  That is only correct while every accumulator
stays in an AGPR: if the register allocator gives the kernel fewer AGPRs, it
moves accumulators through scratch around each asm statement, and those moves
read an MFMA's result with none of the wait states the compiler inserts for
MFMAs it knows about (stale values, no error).  The build therefore asks the
compiler for each kernel's resource usage and fails if such a kernel has
fewer AGPRs than its accumulators need.
"""
from __future__ import annotations

import os
import re
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("api.hip", "gemm.hip", "gemm_ws.hip", "gemv.hip", "probe.hip", "skinny.hip")]
LIBRARY = os.path.join(PKG_DIR, "libgemvtile.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    "-Wno-unused-command-line-argument",
    "-Xclang",
    "-target-feature",
    "-Xclang",
    "-packed-fp32-ops",
    f"-I{os.path.join(REPO_DIR, 'include')}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
_REMARK = re.compile(r"remark:\s+(Function Name|AGPRs|VGPRs|ScratchSize \[bytes/lane\]|VGPRs Spill):\s+(\S+)")


def parse_resource_usage(text: str) -> dict:
    """Kernel name -> {"AGPRs", "VGPRs", "ScratchSize", "VGPRs Spill"} from the
    compiler's kernel-resource-usage remarks."""
    usage: dict = {}
    cur = None
    for m in _REMARK.finditer(text):
        key, val = m.group(1), m.group(2)
        if key == "Function Name":
            cur = usage.setdefault(val, {})
        elif cur is not None:
            cur[key.split(" [")[0]] = int(val)
    return usage


def required_agprs(kernel: str):
    """AGPRs per lane that the inline-asm MFMA accumulators of a kernel need,
    or None for a kernel without such accumulators.

    gemm_kernel<GemmShape<BM, BN, BK, STAGES, WAVES_M, WAVES_N, ..., MI, ...>>
    holds a (BM / WAVES_M) x (BN / WAVES_N) FP32 block per wave, one value
    per lane per 64 outputs; only its MI == 16 form uses inline-asm MFMAs.
    gemm_ws_kernel's consumer waves hold 128 x 64 outputs each."""
    if "gemm_ws_kernel" in kernel:
        return 128 * 64 // 64
    m = re.search(r"gemm_kernelINS_9GemmShapeI((?:L[ib]\d+E)+)E", kernel)
    if not m:
        return None
    args = [int(a) for a in re.findall(r"L[ib](\d+)E", m.group(1))]
    bm, bn, waves_m, waves_n, mi = args[0], args[1], args[4], args[5], args[13]
    if mi != 16:
        return None
    return (bm // waves_m) * (bn // waves_n) // 64


def check_resource_usage(usage: dict) -> list:
    """Kernels whose inline-asm MFMA accumulators do not all fit in AGPRs."""
    bad = []
    for name, u in sorted(usage.items()):
        need = required_agprs(name)
        if need is not None and u.get("AGPRs", 0) < need:
            bad.append(f"{name}: {u.get('AGPRs', 0)} AGPRs for {need} accumulator registers, "
                       f"scratch {u.get('ScratchSize', 0)} bytes/lane")
    return bad


def build_library(output: str = LIBRARY, extra_flags=(), verbose: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, RESOURCE_REMARKS, *extra_flags, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    text = res.stdout + res.stderr
    # hipcc's host pass always warns about the device-only feature flag; the
    # resource remarks are parsed below rather than shown.
    noise = ("is not a recognized feature for this target", "warning generated", "warnings generated",
             "remark:", "kernel-resource-usage")
    lines = text.splitlines()
    msgs = []
    for i, ln in enumerate(lines):
        if any(n in ln for n in noise):
            continue
        # source excerpt and caret under a remark
        if i > 0 and "remark:" in lines[i - 1]:
            continue
        if i > 1 and "remark:" in lines[i - 2] and ln.strip().startswith("|"):
            continue
        msgs.append(ln)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    usage = parse_resource_usage(text)
    bad = check_resource_usage(usage)
    if not usage or bad:
        os.remove(tmp)
        raise RuntimeError("inline-asm MFMA accumulators outside AGPRs (results would be wrong):\n"
                           + ("\n".join(bad) if bad else "no kernel-resource-usage remarks in the compiler output"))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    build_library(verbose="-v" in sys.argv)
    print(LIBRARY)
