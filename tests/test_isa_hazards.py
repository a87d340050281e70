"""The wide prefill kernel's inline-assembly MFMAs and direct-to-LDS loads,
checked in the compiled gfx950 assembly (no GPU needed): no VALU write of an
MFMA operand right before one, no read of an MFMA result right after one, no
VALU write of a load's SGPR operands within 5 wait states and no M0 write
right before a load (the hardware wait states the compiler does not insert
for instructions it cannot see)."""

import pytest

from exact_attention_17_amd import isa_check


@pytest.fixture(scope="module")
def wide_asm():
    return isa_check.compile_to_asm("prefill_wide.hip")


def test_wide_kernel_has_no_inline_mfma_hazards(wide_asm):
    assert "v_mfma_f32_32x32x16_bf16" in wide_asm
    problems = isa_check.check_asm(wide_asm)
    assert problems == [], "\n".join(problems[:20])


def test_wide_kernel_lds_loads_have_their_wait_states(wide_asm):
    assert "offen lds" in wide_asm
    problems = isa_check.check_lds_loads(wide_asm)
    assert problems == [], "\n".join(problems[:20])


def test_lds_load_checker_flags_planted_hazards():
    bad = """
    v_readfirstlane_b32 s12, v3
    s_mov_b32 m0, s40
    ;;#ASMSTART
    buffer_load_dwordx4 v2, s[24:27], s12 offen lds
    ;;#ASMEND
    """
    assert len(isa_check.check_lds_loads(bad)) == 2
    good = """
    v_readfirstlane_b32 s12, v3
    s_nop 3
    s_mov_b32 m0, s40
    ;;#ASMSTART
    s_nop 0
    buffer_load_dwordx4 v2, s[24:27], s12 offen lds
    ;;#ASMEND
    """
    assert isa_check.check_lds_loads(good) == []


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
