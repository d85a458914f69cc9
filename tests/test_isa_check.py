"""The build-time wait-state check of the inline-assembly MFMAs (CPU only).

Each planted hazard below is one of the patterns the check exists to reject;
the clean snippets are the patterns the tile kernel relies on."""

import os

import pytest

from rollout_logprob_consistency_amd import isa_check

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kernel(body_lines):
    body = "\n".join("\t" + l for l in body_lines)
    return (".amdhsa_kernel _Z17score_tile_kernelv\n.end_amdhsa_kernel\n"
            "_Z17score_tile_kernelv:\n" + body + "\n.Lfunc_end0:\n")


ASM_MFMA = [";;#ASMSTART", "v_mfma_f32_16x16x32_bf16 v[20:23], v[0:3], v[4:7], v[20:23]",
            ";;#ASMEND"]


def test_clean_chain_passes():
    lines = ["ds_read_b128 v[0:3], v40", "ds_read_b128 v[4:7], v41", "s_waitcnt lgkmcnt(0)",
             *ASM_MFMA, "v_mfma_f32_16x16x32_bf16 a[0:3], v[0:3], v[4:7], a[0:3]", *ASM_MFMA,
             "s_nop 7", "s_nop 7", "s_nop 7", "v_max_f32_e32 v30, v20, v21"]
    assert isa_check.check_asm(kernel(lines)) == []


def test_valu_write_just_before_is_caught():
    lines = ["v_mov_b64_e32 v[20:21], 0", *ASM_MFMA, "s_nop 7", "s_nop 7", "s_nop 7"]
    assert any("VALU write" in p for p in isa_check.check_asm(kernel(lines)))


def test_valu_write_of_a_source_just_before_is_caught():
    lines = ["v_add_u32_e32 v5, 1, v5", *ASM_MFMA, "s_nop 7", "s_nop 7", "s_nop 7"]
    assert isa_check.check_asm(kernel(lines))


def test_valu_read_of_the_result_too_early_is_caught():
    lines = [*ASM_MFMA, "s_nop 3", "v_mov_b64_e32 v[30:31], v[22:23]"]
    assert any("touches the result" in p for p in isa_check.check_asm(kernel(lines)))


def test_store_of_the_result_too_early_is_caught():
    lines = [*ASM_MFMA, "scratch_store_dwordx4 off, v[20:23], off offset:16"]
    assert any("store" in p for p in isa_check.check_asm(kernel(lines)))


def test_mfma_reading_the_result_as_source_is_caught():
    lines = [*ASM_MFMA, "v_mfma_f32_16x16x32_bf16 a[0:3], v[20:23], v[4:7], a[0:3]"]
    assert isa_check.check_asm(kernel(lines))


def test_enough_wait_states_pass():
    lines = ["v_mov_b64_e32 v[20:21], 0", "s_nop 3", *ASM_MFMA, "s_nop 7", "s_nop 7", "s_nop 3",
             "v_mov_b64_e32 v[30:31], v[22:23]"]
    assert isa_check.check_asm(kernel(lines)) == []


def test_a_kernel_without_asm_mfma_is_reported():
    assert isa_check.check_asm(kernel(["s_endpgm"]))


def test_built_score_kernel_is_clean():
    path = os.path.join(ROOT, "_build", "score.device.s")
    if not os.path.exists(path):
        pytest.skip("no device assembly: the library has not been built here")
    assert isa_check.check_asm(open(path).read()) == []


def cmp_kernel(body_lines):
    body = "\n".join("\t" + l for l in body_lines)
    return "_ZN2lp14compare_kernelEv:\n" + body + "\n.Lfunc_end1:\n"


def test_compare_kernel_without_bpermute_passes():
    lines = ["v_mov_b32_dpp v2, v0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf",
             "ds_swizzle_b32 v3, v0 offset:swizzle(SWAP,16)", "v_readlane_b32 s4, v3, 32"]
    assert isa_check.check_no_bpermute(cmp_kernel(lines)) == []


def test_compare_kernel_with_bpermute_fails():
    lines = ["v_lshlrev_b32_e32 v1, 2, v1", "ds_bpermute_b32 v2, v1, v0"]
    assert isa_check.check_no_bpermute(cmp_kernel(lines))
    assert isa_check.check_no_bpermute("nothing here")     # the kernel must be found


def test_built_compare_kernel_has_no_bpermute():
    # The assembly the last build checked (build() writes it).
    path = os.path.join(ROOT, "_build", "compare.device.s")
    if not os.path.exists(path):
        pytest.skip("no build assembly; run the build first")
    asm = open(path).read()
    assert isa_check.kernel_bodies(asm, "compare_kernel")
    assert isa_check.check_no_bpermute(asm) == []


def dma_kernel(body_lines):
    body = "\n".join("\t" + l for l in body_lines)
    return (".amdhsa_kernel _ZN2lp14compare_kernelEv\n.end_amdhsa_kernel\n"
            "_ZN2lp14compare_kernelEv:\n" + body + "\n.Lfunc_end2:\n")


COPY = [";;#ASMSTART", "s_nop 4", "buffer_load_dwordx4 v18, s[12:15], s8 offen lds", ";;#ASMEND"]


def test_lds_copy_with_its_wait_states_passes():
    lines = ["v_readlane_b32 s15, v63, 19", "s_add_i32 m0, s6, s2", *COPY]
    assert isa_check.check_lds_dma_sgpr(dma_kernel(lines)) == []


def test_spilled_resource_restored_just_before_an_lds_copy_is_caught():
    # the faulting pattern: a v_readlane restoring the resource, then the copy
    # with only one wait state of its own
    lines = ["v_readlane_b32 s15, v63, 19", ";;#ASMSTART", "s_nop 0",
             "buffer_load_dwordx4 v18, s[12:15], s8 offen lds", ";;#ASMEND"]
    assert any("writes an SGPR" in p for p in isa_check.check_lds_dma_sgpr(dma_kernel(lines)))


def test_valu_write_of_the_offset_sgpr_is_caught():
    lines = ["v_cmp_ne_u32_e64 s[8:9], v1, v2", ";;#ASMSTART", "s_nop 1",
             "buffer_load_dword v8, s[20:23], s8 offen lds", ";;#ASMEND"]
    assert isa_check.check_lds_dma_sgpr(dma_kernel(lines))


def test_salu_writes_and_other_registers_pass():
    lines = ["s_lshl_b32 s8, s3, 10", "v_readlane_b32 s30, v63, 2", ";;#ASMSTART", "s_nop 0",
             "buffer_load_dword v8, s[20:23], s8 offen lds", ";;#ASMEND"]
    assert isa_check.check_lds_dma_sgpr(dma_kernel(lines)) == []


@pytest.mark.parametrize("name", ["score.device.s", "compare.device.s"])
def test_built_lds_copies_have_their_wait_states(name):
    path = os.path.join(ROOT, "_build", name)
    if not os.path.exists(path):
        pytest.skip("no build assembly; run the build first")
    assert isa_check.check_lds_dma_sgpr(open(path).read()) == []
