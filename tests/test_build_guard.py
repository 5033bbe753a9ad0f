"""The build's check that inline-asm MFMA accumulators stay in AGPRs.

The remarks below have the form hipcc prints under
-Rpass-analysis=kernel-resource-usage.  The first kernel is the tiled GEMM
with a refill load every MFMA slot, as the compiler once allocated it: 32
AGPRs for 256 accumulator registers and 1552 bytes of scratch per lane.  That
kernel wrote all-zero outputs, and the check must reject it.
"""
from gemv_tile_pipelined_amd import build

SPILLED = "_ZN2gt11gemm_kernelINS_9GemmShapeILi256ELi256ELi64ELi2ELi2ELi2ELb1ELb1ELi1ELi1ELi1ELi1ELi0ELi16ELi2ELi1ELb0ELi0ELb0EEEEEvPKDF16_S4_PDF16_iiiiii"
DEFAULT = "_ZN2gt11gemm_kernelINS_9GemmShapeILi256ELi256ELi64ELi2ELi2ELi2ELb1ELb1ELi4ELi1ELi1ELi1ELi0ELi16ELi2ELi1ELb0ELi0ELb0EEEEEvPKDF16_S4_PDF16_iiiiii"
EIGHT_WAVES = "_ZN2gt11gemm_kernelINS_9GemmShapeILi256ELi256ELi64ELi2ELi2ELi4ELb1ELb1ELi4ELi1ELi1ELi1ELi0ELi16ELi2ELi1ELb0ELi0ELb0EEEEEvPKDF16_S4_PDF16_iiiiii"
MI32_ONE_STAGE = "_ZN2gt11gemm_kernelINS_9GemmShapeILi256ELi256ELi64ELi1ELi2ELi2ELb1ELb1ELi1ELi1ELi1ELi1ELi0ELi32ELi1ELi0ELb0ELi0ELb0EEEEEvPKDF16_S4_PDF16_iiiiii"
WS = "_ZN2gt14gemm_ws_kernelILi3ELi0EEEvPKDF16_S2_PDF16_iiiiii"
GEMV = "_ZN2gt11gemv_kernelILi2ELi8ELi4ELb1ELb1ELi0ELi1ELin1EEEvPKvS2_Pviii"


def _remarks(name, agprs, vgprs, scratch, spill=0):
    loc = "gemm.hip:300:1: remark: "
    tail = " [-Rpass-analysis=kernel-resource-usage]"
    return "\n".join([
        f"{loc}Function Name: {name}{tail}",
        "  300 | __global__ void f() {",
        "      | ^",
        f"{loc}    TotalSGPRs: 80{tail}",
        f"{loc}    VGPRs: {vgprs}{tail}",
        f"{loc}    AGPRs: {agprs}{tail}",
        f"{loc}    ScratchSize [bytes/lane]: {scratch}{tail}",
        f"{loc}    Dynamic Stack: False{tail}",
        f"{loc}    Occupancy [waves/SIMD]: 1{tail}",
        f"{loc}    SGPRs Spill: 0{tail}",
        f"{loc}    VGPRs Spill: {spill}{tail}",
        f"{loc}    LDS Size [bytes/block]: 131072{tail}",
    ])


def test_required_agprs():
    assert build.required_agprs(DEFAULT) == 256  # 128 x 128 per wave
    assert build.required_agprs(EIGHT_WAVES) == 128  # 128 x 64 per wave
    assert build.required_agprs(WS) == 128
    assert build.required_agprs(MI32_ONE_STAGE) is None  # compiler's own MFMAs
    assert build.required_agprs(GEMV) is None


def test_parse_and_check():
    text = "\n".join([
        _remarks(SPILLED, 32, 208, 1552),
        _remarks(DEFAULT, 256, 396, 0),
        _remarks(EIGHT_WAVES, 128, 232, 0),
        _remarks(MI32_ONE_STAGE, 256, 512, 32, spill=7),
        _remarks(WS, 128, 128, 16, spill=3),
        _remarks(GEMV, 0, 40, 0),
    ])
    usage = build.parse_resource_usage(text)
    assert set(usage) == {SPILLED, DEFAULT, EIGHT_WAVES, MI32_ONE_STAGE, WS, GEMV}
    assert usage[SPILLED] == {"VGPRs": 208, "AGPRs": 32, "ScratchSize": 1552, "VGPRs Spill": 0}
    bad = build.check_resource_usage(usage)
    assert len(bad) == 1 and bad[0].startswith(SPILLED) and "32 AGPRs for 256" in bad[0]


def test_check_flags_one_agpr_short():
    usage = build.parse_resource_usage(_remarks(EIGHT_WAVES, 127, 232, 0))
    assert len(build.check_resource_usage(usage)) == 1
