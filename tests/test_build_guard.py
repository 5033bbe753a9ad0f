"""The build's checks that inline-asm MFMA accumulators stay in place.

The remarks below have the form hipcc prints under
-Rpass-analysis=kernel-resource-usage.  The first kernel is the tiled GEMM
with a refill load every MFMA slot, as the compiler once allocated it: 32
AGPRs for 256 accumulator registers and 1552 bytes of scratch per lane.  That
kernel wrote all-zero outputs, and the check must reject it.

The assembly snippets reproduce, in miniature, what the compiler emitted for
a GEMM variant that kept all its AGPRs but spilled VGPRs: accumulators copied
out a few instructions after the MFMA that writes them, and written back one
instruction before the MFMA that reads them.  That variant gave wrong bits;
the scan must flag both patterns and accept the padded reads the kernels
write themselves.
"""
from gemv_tile_pipelined_amd import build

# GemmShape<BM, BN, BK, STAGES, WAVES_M, WAVES_N, SWIZZLE, PERSISTENT,
# DMA_STRIDE, MI, READ_STRIDE, DMA_OFFSET, DTYPE>
SPILLED = "_ZN2gt11gemm_kernelINS_9GemmShapeILi256ELi256ELi64ELi2ELi2ELi2ELb1ELb1ELi1ELi16ELi2ELi1ELi0EEELi0EEEvPKDF16_S4_PDF16_iiiiiiPKtiPfi"
DEFAULT = "_ZN2gt11gemm_kernelINS_9GemmShapeILi256ELi256ELi64ELi2ELi2ELi2ELb1ELb1ELi4ELi16ELi2ELi1ELi0EEELi0EEEvPKDF16_S4_PDF16_iiiiiiPKtiPfi"
EIGHT_WAVES = "_ZN2gt11gemm_kernelINS_9GemmShapeILi256ELi256ELi64ELi2ELi2ELi4ELb1ELb1ELi4ELi16ELi2ELi1ELi0EEELi0EEEvPKDF16_S4_PDF16_iiiiiiPKtiPfi"
MI32_ONE_STAGE = "_ZN2gt11gemm_kernelINS_9GemmShapeILi256ELi256ELi64ELi1ELi2ELi2ELb1ELb1ELi1ELi32ELi1ELi0ELi0EEELi0EEEvPKDF16_S4_PDF16_iiiiiiPKtiPfi"
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


def test_check_flags_spilled_fragments():
    # all AGPRs in place, but the operand fragments of a partly unrolled K
    # loop spilled to scratch (as a too-low unroll limit once produced)
    usage = build.parse_resource_usage(_remarks(DEFAULT, 256, 512, 1040, spill=120))
    bad = build.check_resource_usage(usage)
    assert len(bad) == 1 and "scratch 1040" in bad[0]


def test_parse_remarks_with_location_after_tag():
    """With -save-temps the backend prints 'remark: file:line:col: Key: value'."""
    text = "\n".join([
        f"remark: /src/gemm.hip:44:0: Function Name: {WS} [-Rpass-analysis=kernel-resource-usage]",
        "remark: /src/gemm.hip:44:0:     VGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "remark: /src/gemm.hip:44:0:     AGPRs: 128 [-Rpass-analysis=kernel-resource-usage]",
        "remark: /src/gemm.hip:44:0:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]",
        "remark: /src/gemm.hip:44:0:     VGPRs Spill: 3 [-Rpass-analysis=kernel-resource-usage]",
    ])
    assert build.parse_resource_usage(text) == {WS: {"VGPRs": 128, "AGPRs": 128, "ScratchSize": 16, "VGPRs Spill": 3}}


def _asm(name, lines):
    """A device-assembly function in the layout hipcc writes; lines starting
    with '!' are wrapped in inline-asm markers."""
    out = [f"{name}:                 ; @{name}", "; %bb.0:"]
    for ln in lines:
        if ln.startswith("!"):
            out += ["\t;;#ASMSTART", "\t" + ln[1:], "\t;;#ASMEND"]
        else:
            out.append("\t" + ln)
    out += [".Lfunc_end0:", f"\t.size\t{name}, .Lfunc_end0-{name}"]
    return "\n".join(out) + "\n"


MFMA = "!v_mfma_f32_16x16x32_f16 a[252:255], v[60:63], v[56:59], a[252:255]"


def test_hazard_scan_accepts_padded_reads():
    # the kernels' own pattern: MFMAs, 24 wait states of padding, then reads
    ok = _asm(DEFAULT, [MFMA, "!v_mfma_f32_16x16x32_f16 a[248:251], v[4:7], v[56:59], a[248:251]",
                        "!s_nop 7", "!s_nop 7", "!s_nop 7", "v_accvgpr_read_b32 v0, a252", "v_accvgpr_read_b32 v4, a248"])
    assert build.scan_mfma_hazards(ok) == []


def test_hazard_scan_flags_early_accumulator_read():
    # as the compiler emitted under register pressure: an accumulator copied
    # out a few instructions after the MFMA that writes it
    bad = _asm(DEFAULT, [MFMA, "v_add_u32_e32 v96, s9, v118", "ds_read_b128 v[104:107], v96",
                         "s_add_i32 s12, s11, 0x8000", "s_mov_b32 m0, s12", "s_nop 0",
                         "v_accvgpr_read_b32 v0, a252"])
    found = build.scan_mfma_hazards(bad)
    assert len(found) == 1 and "v_accvgpr_read_b32 v0, a252" in found[0]


def test_hazard_scan_flags_late_accumulator_restore():
    # an accumulator written back one instruction before the MFMA reads it
    bad = _asm(DEFAULT, ["v_accvgpr_write_b32 a255, v167", MFMA])
    found = build.scan_mfma_hazards(bad)
    assert len(found) == 1 and "writes a source" in found[0]
    # and an operand register written by a VALU op right before the MFMA
    bad2 = _asm(DEFAULT, ["v_mov_b32_e32 v58, v200", MFMA])
    assert len(build.scan_mfma_hazards(bad2)) == 1
    # a VGPR that shares its number with the MFMA's accumulator is another register
    ok = _asm(DEFAULT, ["v_add_u32_e32 v253, s55, v94", MFMA])
    assert build.scan_mfma_hazards(ok) == []


LDS_DMA = "!s_mov_b32 m0, s12\n\ts_nop 0\n\tbuffer_load_dwordx4 v118, s[16:19], 0 offen lds"


def test_m0_scan_accepts_inline_only_m0():
    ok = _asm(DEFAULT, [LDS_DMA, MFMA, "s_add_i32 s12, s12, 0x1000", LDS_DMA, "ds_read_b128 v[4:7], v96"])
    assert build.scan_m0_uses(ok) == []


def test_m0_scan_flags_compiler_m0_use():
    # the compiler keeps a value in M0 across the inline asm that overwrites it
    bad = _asm(DEFAULT, ["s_mov_b32 m0, s40", LDS_DMA, "v_movrels_b32_e32 v1, v8"])
    found = build.scan_m0_uses(bad)
    assert len(found) == 2 and "s_mov_b32 m0, s40" in found[0] and "v_movrels" in found[1]
    # a compiler LDS-DMA (reads M0 implicitly) and an explicit read of M0
    bad2 = _asm(DEFAULT, [LDS_DMA, "buffer_load_dword v1, s[16:19], 0 offen lds", "s_mov_b32 s3, m0"])
    assert len(build.scan_m0_uses(bad2)) == 2
    # a kernel without inline M0 writes is not scanned
    assert build.scan_m0_uses(_asm(GEMV, ["s_mov_b32 m0, s40", "ds_gws_init v0"])) == []


def test_hazard_scan_skips_compiler_mfmas_and_other_kernels():
    # an MFMA the compiler wrote (no inline-asm markers) is padded by the
    # compiler itself; kernels without inline-asm MFMAs are not scanned
    compiler = _asm(MI32_ONE_STAGE, ["v_mfma_f32_32x32x16_f16 a[64:79], v[32:35], v[24:27], a[64:79]",
                                     "v_accvgpr_write_b32 a64, 0"])
    assert build.scan_mfma_hazards(compiler) == []
    other = _asm(GEMV, [MFMA, "v_accvgpr_read_b32 v0, a252"])
    assert build.scan_mfma_hazards(other) == []
