"""The wide prefill kernel's inline-assembly MFMAs, checked in the compiled
gfx950 assembly (no GPU needed): no VALU write of an operand right before one,
no read of a result right after one (the hardware wait states the compiler
does not insert for instructions it cannot see)."""

import pytest

from exact_attention_17_amd import isa_check


@pytest.fixture(scope="module")
def wide_asm():
    return isa_check.compile_to_asm("prefill_wide.hip")


def test_wide_kernel_has_no_inline_mfma_hazards(wide_asm):
    assert "v_mfma_f32_32x32x16_bf16" in wide_asm
    problems = isa_check.check_asm(wide_asm)
    assert problems == [], "\n".join(problems[:20])


def test_checker_flags_planted_hazards():
    """A VALU write of an MFMA operand one instruction before it, and a read of
    its result right after it, are both reported; the same with enough wait
    states between is not."""
    bad = """
    v_mov_b32 v8, v1
    ;;#ASMSTART
    v_mfma_f32_32x32x16_bf16 v[20:35], v[8:11], a[0:3], v[20:35]
    ;;#ASMEND
    v_add_f32 v40, v21, v22
    """
    problems = isa_check.check_asm(bad)
    assert len(problems) == 2
    good = """
    v_mov_b32 v8, v1
    s_nop 2
    ;;#ASMSTART
    v_mfma_f32_32x32x16_bf16 v[20:35], v[8:11], a[0:3], v[20:35]
    ;;#ASMEND
    s_nop 7
    s_nop 7
    s_nop 3
    v_add_f32 v40, v21, v22
    """
    assert isa_check.check_asm(good) == []
