"""CPU-only: the build's check of the compiler's per-kernel resource remarks (no scratch in
any kernel, 4 waves per SIMD for the GEMMs launched two blocks per CU) flags what it should,
on remark lines in the compiler's format, and passes the kernels as they are built."""

from block_diffusion_lm_router_amd import build


def remarks(name, scratch, waves):
    loc = "csrc/moe_w4a16.hip:763:1: remark:"
    return "\n".join([
        f"{loc} Function Name: {name} [-Rpass-analysis=kernel-resource-usage]",
        f"{loc}     VGPRs: 116 [-Rpass-analysis=kernel-resource-usage]",
        f"{loc}     ScratchSize [bytes/lane]: {scratch} [-Rpass-analysis=kernel-resource-usage]",
        f"{loc}     Occupancy [waves/SIMD]: {waves} [-Rpass-analysis=kernel-resource-usage]",
    ])


GEMM = "_ZN2bd12_GLOBAL__N_119w4a16_packed_kernelILb1ELi22ELb0EEEvNS0_8GemmArgsE"
DOWN = "_ZN2bd12_GLOBAL__N_126w4a16_down_resident_kernelILb0EEEvNS0_8GemmArgsE"
OTHER = "_ZN2bd12_GLOBAL__N_114rmsnorm_kernelEPKtS2_iifPtPKi"


def test_clean_remarks_pass():
    assert build.check_resources(remarks(GEMM, 0, 4) + "\n" + remarks(OTHER, 0, 1)) == []


def test_scratch_is_flagged_for_any_kernel():
    problems = build.check_resources(remarks(OTHER, 8, 1))
    assert len(problems) == 1 and "scratch" in problems[0] and OTHER in problems[0]


def test_low_occupancy_is_flagged_for_the_gemms_only():
    assert build.check_resources(remarks(OTHER, 0, 1)) == []
    for name in (GEMM, DOWN):
        problems = build.check_resources(remarks(name, 0, 3))
        assert len(problems) == 1 and "waves per SIMD" in problems[0] and name in problems[0]


def test_each_kernel_is_judged_on_its_own_lines():
    text = remarks(GEMM, 0, 4) + "\n" + remarks(DOWN, 0, 2) + "\n" + remarks(OTHER, 4, 8)
    problems = build.check_resources(text)
    assert len(problems) == 2
    assert any(DOWN in p for p in problems) and any(OTHER in p for p in problems)
