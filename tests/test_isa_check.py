"""The wait-state checker that guards the assembly MFMAs of the 64-row-wave forward kernel."""
from scaled_dot_product_08_amd import isa_check

MFMA = "v_mfma_f32_32x32x16_bf16 a[0:15], v[0:3], v[4:7], a[0:15]"


def _asm(*lines):
    return "\n".join("\t" + l for l in lines)


def test_clean_sequence_passes():
    text = _asm("v_cvt_pk_bf16_f32 v4, v8, v9", "s_nop 1", MFMA, "s_nop 7", "s_nop 7",
                "v_accvgpr_read_b32 v10, a3")
    assert isa_check.check(text) == []


def test_operand_written_too_late_is_found():
    text = _asm("v_cvt_pk_bf16_f32 v5, v8, v9", "s_nop 0", MFMA)
    bad = isa_check.check(text)
    assert len(bad) == 1 and "writes an operand" in bad[0]


def test_operand_write_two_states_earlier_is_fine():
    assert isa_check.check(_asm("v_mov_b32 v1, v9", "v_add_f32 v20, v21, v22", "s_nop 0", MFMA)) == []


def test_accumulator_read_too_early_is_found():
    for reader in ("v_accvgpr_read_b32 v10, a15", "v_accvgpr_mov_b32 a20, a2",
                   "scratch_store_dwordx4 off, a[0:3], off offset:16"):
        bad = isa_check.check(_asm(MFMA, "s_nop 7", reader))
        assert len(bad) == 1 and "accesses an accumulator" in bad[0], reader


def test_unrelated_accumulator_is_fine():
    assert isa_check.check(_asm(MFMA, "v_accvgpr_read_b32 v10, a16")) == []


def test_compiler_mfma_is_not_checked():
    # VGPR-destination MFMAs are the compiler's own; it inserts their wait states.
    text = _asm("v_mov_b32 v1, v9", "v_mfma_f32_32x32x16_bf16 v[16:31], v[0:3], v[4:7], 0",
                "v_add_f32 v20, v16, v17")
    assert isa_check.check(text) == []


def test_kernel_split():
    text = "_Zfoo_w64_a:\n" + _asm(MFMA, "s_endpgm") + "\n_Zbar:\n" + _asm("s_endpgm")
    ks = isa_check.kernels(text, "w64")
    assert list(ks) == ["_Zfoo_w64_a"] and MFMA in ks["_Zfoo_w64_a"]
