"""Build the gfx950 library libgemvtile.so in-tree with hipcc.

Usage: python -m gemv_tile_pipelined_amd.build   (or call build_library()).
The library is compiled for gfx950 only.  Packed-FP32 instructions are
disabled for the device code (-packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.
"""
from __future__ import annotations

import os
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


def build_library(output: str = LIBRARY, extra_flags=(), verbose: bool = False) -> str:
    tmp = output + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra_flags, *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass always warns about the device-only feature flag.
    noise = ("is not a recognized feature for this target", "warning generated", "warnings generated")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    build_library(verbose="-v" in sys.argv)
    print(LIBRARY)
