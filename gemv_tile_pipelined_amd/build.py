"""Build the gfx950 library libgemvtile.so in-tree with hipcc.

Usage: python -m gemv_tile_pipelined_amd.build   (or call build_library()).
The library is compiled for gfx950 only.  Packed-FP32 instructions are
disabled for the device code (-packed-fp32-ops); hipcc's host pass warns that
it does not know that feature, which is harmless.

The GEMM kernels issue their 16x16x32 MFMAs as inline asm with the
accumulators bound to AGPRs.  That is only correct while every accumulator
stays in place: if register pressure makes the allocator move accumulators
(to scratch, or to other registers), its moves read an MFMA's result with
none of the wait states the compiler inserts for MFMAs it knows about, and
the kernel computes stale values with no error.  The build therefore checks
the code it produced, in two ways, and fails if either finds a problem:
  * the compiler's resource-usage remarks: every kernel with inline-asm
    MFMAs has at least as many AGPRs as its accumulators need;
  * the device assembly of those kernels (kept from the same compilation
    with -save-temps): no instruction other than an MFMA reads or writes an
    MFMA's destination registers within MFMA_RESULT_WAIT wait states of it,
    and no VALU instruction writes an MFMA source register within
    VALU_TO_MFMA_WAIT wait states before it.

The direct-to-LDS tile loads are inline asm that write M0 (the LDS address)
and use it in the same statement.  The compiler reserves M0 for its own use
and does not know these statements change it, so they are only safe while
the compiler keeps no value in M0 across them.  The build checks that too:
in every kernel whose inline asm writes M0, no instruction the compiler
emitted reads or writes M0, explicitly or implicitly (scan_m0_uses).
"""
from __future__ import annotations

import glob
import os
import re
import subprocess
import sys
import tempfile

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
REPO_DIR = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("api.hip", "gemm.hip", "gemm_plain.hip", "gemm_ws.hip", "gemv.hip", "skinny.hip")]
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
    # The pipelined GEMM K loop (ring.hpp) is written as fully unrolled loops
    # over MFMA slots; its unrolled size exceeds the compiler's default limit
    # for `#pragma unroll`, and a partly unrolled loop indexes the fragment
    # arrays at run time, which puts them in scratch memory.
    "-mllvm",
    "-pragma-unroll-threshold=200000",
    f"-I{os.path.join(REPO_DIR, 'include')}",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


RESOURCE_REMARKS = "-Rpass-analysis=kernel-resource-usage"
# Either "file:line:col: remark: Key: value" or, when the backend runs as a
# separate step (-save-temps), "remark: file:line:col: Key: value".
_REMARK = re.compile(r"remark:\s+(?:\S+:\d+:\d+:\s+)?(Function Name|AGPRs|VGPRs|ScratchSize \[bytes/lane\]|VGPRs Spill):"
                     r"\s+(\S+)")


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

    gemm_kernel<GemmShape<BM, BN, BK, STAGES, WAVES_M, WAVES_N, SWIZZLE,
    PERSISTENT, DMA_STRIDE, MI, ...>> holds a (BM / WAVES_M) x (BN / WAVES_N) FP32 block per wave, one value
    per lane per 64 outputs; only its MI == 16 form uses inline-asm MFMAs.
    gemm_ws_kernel's consumer waves hold 128 x 64 outputs each."""
    if "gemm_ws_kernel" in kernel:
        return 128 * 64 // 64
    m = re.search(r"gemm_kernelINS_9GemmShapeI((?:L[ib]\d+E)+)E", kernel)
    if not m:
        return None
    args = [int(a) for a in re.findall(r"L[ib](\d+)E", m.group(1))]
    bm, bn, waves_m, waves_n, mi = args[0], args[1], args[4], args[5], args[9]
    if mi != 16:
        return None
    return (bm // waves_m) * (bn // waves_n) // 64


# Scratch bytes per lane an inline-asm MFMA kernel may use.  A few spilled
# dwords outside the K loop occur (the fused-bias epilogue spills 28 bytes of
# addresses); a partly unrolled K loop puts its operand fragment arrays in
# scratch (hundreds of bytes), which this limit rejects.
MAX_SCRATCH_BYTES = 64


def check_resource_usage(usage: dict) -> list:
    """Kernels whose inline-asm MFMA accumulators do not all fit in AGPRs, or
    that keep more than MAX_SCRATCH_BYTES per lane in scratch memory."""
    bad = []
    for name, u in sorted(usage.items()):
        need = required_agprs(name)
        if need is None:
            continue
        if u.get("AGPRs", 0) < need or u.get("ScratchSize", 0) > MAX_SCRATCH_BYTES:
            bad.append(f"{name}: {u.get('AGPRs', 0)} AGPRs for {need} accumulator registers, "
                       f"scratch {u.get('ScratchSize', 0)} bytes/lane")
    return bad


# Wait states counted by scan_mfma_hazards: each instruction is one, `s_nop N`
# is N + 1.  The 16x16x32 MFMA's result needs fewer than MFMA_RESULT_WAIT
# before another instruction may touch it; the kernels pad 24 before reading
# their accumulators.
MFMA_RESULT_WAIT = 16
VALU_TO_MFMA_WAIT = 2
# Kernels whose MFMAs are inline asm (the compiler pads its own MFMAs).
INLINE_MFMA_KERNELS = ("gemm_kernel", "gemm_ws_kernel")

_FUNC_START = re.compile(r"^(_Z\S+):\s*(;.*)?$")
_AREG = re.compile(r"(?<![\w.])a(?:\[(\d+):(\d+)\]|(\d+)(?![\w]))")
_VREG = re.compile(r"(?<![\w.])v(?:\[(\d+):(\d+)\]|(\d+)(?![\w]))")


def _regs(pattern, text: str) -> set:
    """Registers named in `text`, as (kind, number) with kind "a" or "v"."""
    kind = "a" if pattern is _AREG else "v"
    out = set()
    for m in pattern.finditer(text):
        if m.group(3) is not None:
            out.add((kind, int(m.group(3))))
        else:
            out.update((kind, r) for r in range(int(m.group(1)), int(m.group(2)) + 1))
    return out


def _functions(asm: str):
    """(name, [(instruction, from_inline_asm)]) for every function in a device
    .s file; the compiler brackets inline asm with ;;#ASMSTART / ;;#ASMEND."""
    name, body, in_asm = None, [], False
    for line in asm.splitlines():
        m = _FUNC_START.match(line)
        if m:
            name, body, in_asm = m.group(1), [], False
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            yield name, body
            name = None
            continue
        stripped = line.strip()
        if stripped.startswith(";;#ASMSTART"):
            in_asm = True
        elif stripped.startswith(";;#ASMEND"):
            in_asm = False
        code = line.split(";")[0].strip()
        if code and not code.startswith(".") and not code.endswith(":"):
            body.append((code, in_asm))


def scan_mfma_hazards(asm: str, kernels=INLINE_MFMA_KERNELS) -> list:
    """Places in the listed kernels where code touches the result of an
    inline-asm MFMA, or writes its sources, too soon (see the module
    docstring).  MFMAs the compiler wrote itself are left to its own hazard
    padding.  The scan follows the listing's order, i.e. fall-through paths;
    an inline-asm MFMA is never the last instruction before a branch in
    these kernels' hot loops, whose bodies are straight-line."""
    bad = []
    for name, body in _functions(asm):
        if not any(k in name for k in kernels):
            continue
        pending = []  # [wait states since issue, destination AGPRs, text] of recent inline-asm MFMAs
        recent_writes = []  # [wait states since issue, written VGPRs/AGPRs, text] of recent VALU ops
        for ins, from_asm in body:
            op = ins.split()[0]
            if op.startswith("v_mfma") and from_asm:
                ops = [o.strip() for o in ins.split(None, 1)[1].split(",")]
                dst, srcs = _regs(_AREG, ops[0]), _regs(_VREG, ops[1]) | _regs(_VREG, ops[2])
                src_c = _regs(_AREG, ops[3]) if len(ops) > 3 else set()
                for age, regs, text in recent_writes:
                    if age < VALU_TO_MFMA_WAIT and (regs & srcs or regs & src_c):
                        bad.append(f"{name}: '{text}' writes a source of '{ins}' {age} wait states before it")
                step, entry = 1, [0, dst, ins]
            elif op.startswith("v_mfma"):
                step, entry = 1, None
            else:
                step = int(ins.split()[1], 0) + 1 if op == "s_nop" else 1
                touched = _regs(_AREG, ins)
                for age, regs, text in pending:
                    if age < MFMA_RESULT_WAIT and touched & regs:
                        bad.append(f"{name}: '{ins}' touches the result of '{text}' {age} wait states after it")
                entry = None
                if op.startswith("v_") and len(ins.split()) > 1:
                    first = ins.split(None, 1)[1].split(",")[0]
                    written = _regs(_VREG, first) | _regs(_AREG, first)
                    if written:
                        recent_writes.append([0, written, ins])
            for lst in (pending, recent_writes):
                for e in lst:
                    e[0] += step
            pending[:] = [e for e in pending if e[0] < MFMA_RESULT_WAIT]
            recent_writes[:] = [e for e in recent_writes if e[0] < VALU_TO_MFMA_WAIT]
            if entry is not None:
                pending.append(entry)
    return bad


def _compile_one(src: str, work: str, extra_flags, verbose: bool):
    """Compile one source to an object in its own directory (so -save-temps
    keeps that source's device assembly apart); returns (object, compiler
    output, return code, {assembly name: text})."""
    name = os.path.splitext(os.path.basename(src))[0]
    wdir = os.path.join(work, name)
    os.makedirs(wdir, exist_ok=True)
    obj = os.path.join(wdir, name + ".o")
    flags = [f for f in HIPCC_FLAGS if f != "-shared"]
    cmd = [hipcc(), *flags, "-c", RESOURCE_REMARKS, "-save-temps=cwd", *extra_flags, src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True, cwd=wdir)
    asm = {os.path.basename(f): open(f).read() for f in glob.glob(os.path.join(wdir, "*-hip-amdgcn-*.s"))}
    return obj, res.stdout + res.stderr, res.returncode, asm


# Instructions that read M0 without naming it (gfx9 family): indexed register
# moves, messages, GWS and ordered-count LDS operations, LDS-DMA loads,
# address-by-lane LDS operations and interpolation.
_M0_IMPLICIT = re.compile(r"^(s_movrel|v_movrel|s_sendmsg|ds_gws_|ds_ordered_count|ds_append|ds_consume|"
                          r"ds_read_addtid|ds_write_addtid|v_interp|s_ttracedata|global_load_lds|"
                          r"scratch_load_lds)")
_M0_OPERAND = re.compile(r"(?<![\w.])m0(?![\w])")


def _uses_m0(ins: str) -> bool:
    op = ins.split()[0]
    if _M0_IMPLICIT.match(op):
        return True
    if op.startswith("buffer_load") and re.search(r"\blds\b", ins):
        return True
    return bool(_M0_OPERAND.search(ins.split(None, 1)[1] if len(ins.split(None, 1)) > 1 else ""))


def scan_m0_uses(asm: str) -> list:
    """Compiler-emitted instructions that read or write M0 in a function whose
    inline asm writes M0 (see the module docstring)."""
    bad = []
    for name, body in _functions(asm):
        if not any(from_asm and _M0_OPERAND.search(ins) and ins.split()[0].startswith("s_mov") for ins, from_asm in body):
            continue
        for ins, from_asm in body:
            if not from_asm and _uses_m0(ins):
                bad.append(f"{name}: compiler-emitted '{ins}' uses M0, which inline asm in this kernel writes")
    return bad


def build_library(output: str = LIBRARY, extra_flags=(), verbose: bool = False) -> str:
    from concurrent.futures import ThreadPoolExecutor

    tmp = output + ".tmp"
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with tempfile.TemporaryDirectory(prefix="gemvtile_build_") as work:
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda s: _compile_one(s, work, extra_flags, verbose), SOURCES))
        text = "".join(r[1] for r in results)
        asm = {}
        for r in results:
            asm.update(r[3])
        failed = [os.path.basename(s) for s, r in zip(SOURCES, results) if r[2] != 0]
        if not failed:
            link = [hipcc(), f"--offload-arch={ARCH}", "-fPIC", "-shared", *[r[0] for r in results], "-o", tmp]
            if verbose:
                print(" ".join(link), flush=True)
            lres = subprocess.run(link, capture_output=True, text=True, cwd=work)
            text += lres.stdout + lres.stderr
            if lres.returncode != 0:
                failed.append("link")
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
    if failed:
        raise RuntimeError(f"hipcc failed ({', '.join(failed)}):\n" + "\n".join(msgs))
    usage = parse_resource_usage(text)
    bad = check_resource_usage(usage)
    if not usage:
        bad.append("no kernel-resource-usage remarks in the compiler output")
    if len(asm) != len(SOURCES):
        bad.append(f"expected {len(SOURCES)} device assembly files from -save-temps, found {sorted(asm)}")
    for fname, text_s in sorted(asm.items()):
        bad += scan_mfma_hazards(text_s)
        bad += scan_m0_uses(text_s)
    if bad:
        os.remove(tmp)
        raise RuntimeError("inline-asm MFMA accumulators or M0 not left to the inline asm (results would be wrong):\n"
                           + "\n".join(bad[:20]) + (f"\n... {len(bad) - 20} more" if len(bad) > 20 else ""))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, output)
    return output


if __name__ == "__main__":
    build_library(verbose="-v" in sys.argv)
    print(LIBRARY)
