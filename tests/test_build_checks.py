"""CPU checks of the library build's guard on the attention kernels' assembly: the
output accumulators live in the fixed accumulation registers a0..a63, owned by inline
assembly, so the build must reject any compiler-generated instruction that names them,
a kernel granted fewer than 64 accumulation registers, and packed-fp32 VALU
instructions (disabled for the whole library)."""
import pytest

from rolling_window_attention_amd import build as B

K = B.ATTN_KERNEL_PREFIX + "ILb0EEEvNS_8AttnArgsE"


def _asm(body, nfv=256, acc=160, kernel=K):
    return f"""	.text
{kernel}:
	s_load_dwordx2 s[0:1], s[4:5], 0x0
	;;#ASMSTART
	s_nop 1
	v_mfma_f32_32x32x16_bf16 a[0:15], v[2:5], v[6:9], a[0:15]
	;;#ASMEND
{body}
	s_endpgm
.Lfunc_end0:
	.amdhsa_kernel {kernel}
		.amdhsa_next_free_vgpr {nfv}
		.amdhsa_accum_offset {acc}
	.end_amdhsa_kernel
"""


def test_clean_kernel_passes():
    B.check_attention_asm(_asm("\tv_accvgpr_write_b32 a64, v1\n\ts_nop 1\n"
                               "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[2:5], a[64:67], v[0:15]"))


@pytest.mark.parametrize("body", [
    "\tv_accvgpr_write_b32 a5, v1",
    "\tv_accvgpr_read_b32 v1, a63",
    "\tbuffer_load_dwordx4 a[60:63], v1, s[0:3], 0 offen",
    "\tds_write_b128 v1, a[0:3]",
    "\tv_pk_fma_f32 v[0:1], v[2:3], v[4:5], v[6:7]",
])
def test_violations_are_rejected(body):
    with pytest.raises(RuntimeError):
        B.check_attention_asm(_asm(body))


def test_too_few_accumulation_registers_rejected():
    with pytest.raises(RuntimeError):
        B.check_attention_asm(_asm("", nfv=256, acc=224))


def test_other_kernels_may_use_accumulation_registers():
    # only the attention kernels own a0..a63
    txt = _asm("") + _asm("\tv_accvgpr_write_b32 a5, v1", kernel="_ZN6rfattn17window_attn_fixupENS_8AttnArgsE")
    B.check_attention_asm(txt)


def test_missing_kernels_rejected():
    with pytest.raises(RuntimeError):
        B.check_attention_asm(_asm("", kernel="_ZN6rfattn5otherEv"))


def test_agpr_alloc_attribute_edit():
    ll = ('define protected amdgpu_kernel void @' + K + '(ptr %0) local_unnamed_addr #2 comdat {\n'
          'define protected amdgpu_kernel void @_ZN6rfattn17window_attn_fixupENS_8AttnArgsE(ptr %0) #0 {\n'
          'attributes #0 = { "amdgpu-agpr-alloc"="0" nounwind }\n'
          'attributes #2 = { "amdgpu-agpr-alloc"="0" convergent }\n')
    out = B.set_agpr_alloc(ll, 96)
    assert 'attributes #2 = { "amdgpu-agpr-alloc"="96" convergent }' in out
    assert 'attributes #0 = { "amdgpu-agpr-alloc"="0" nounwind }' in out


# ---- wait-state hazards around inline-assembly MFMAs ---------------------------------
MF = "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]"


def _hz(body):
    return B.mfma_hazards(body.split("\n"), "k")


def test_reading_an_mfma_result_too_early_is_rejected():
    assert _hz(MF + "\n\tv_mov_b32 v30, v3")                            # right after
    assert _hz(MF + "\n\ts_nop 7\n\tv_max3_f32 v30, v1, v2, v3")        # 9 wait states
    assert not _hz(MF + "\n\ts_nop 7\n\ts_nop 3\n\tv_mov_b32 v30, v3")  # 13
    assert not _hz(MF + "\n\tv_mov_b32 v30, v40")                       # other registers


def test_mfma_chains_and_valu_to_mfma():
    # accumulating into the same registers: interlocked
    assert not _hz(MF + "\n" + MF)
    # an MFMA result as the A operand of the next MFMA: hazard
    assert _hz(MF + "\n\tv_mfma_f32_32x32x16_bf16 v[40:55], v[0:3], v[20:23], v[40:55]")
    # VALU write feeding an MFMA operand needs two wait states
    assert _hz("\tv_cvt_pk_bf16_f32 v20, v1, v2\n" + MF)
    assert not _hz("\tv_cvt_pk_bf16_f32 v20, v1, v2\n\ts_nop 1\n" + MF)


def test_hazard_across_a_branch_is_found():
    body = MF + "\n\ts_cbranch_scc1 .LBB0_2\n\ts_nop 7\n\ts_nop 7\n.LBB0_2:\n\tv_mov_b32 v30, v5"
    assert _hz(body)  # the taken path reaches the read without the s_nops


def test_check_attention_asm_reports_hazards():
    with pytest.raises(RuntimeError):
        B.check_attention_asm(_asm("\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], a[64:67], v[0:15]\n"
                                   "\tv_max3_f32 v30, v1, v2, v3"))
