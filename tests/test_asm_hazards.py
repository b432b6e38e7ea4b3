"""Wait states around the inline-assembly MFMAs of the built library (CPU: disassembly only).

The checker is pinned first on small listings in llvm-objdump's format whose verdict follows from
the two rules (two wait states between a VALU write and an MFMA reading the register; twelve between
an 8-pass MFMA's write and any other access to its destination), then run over every gfx950 code
object of the built library.
"""
import os

import pytest

from attention_backward_fa_amd import binding as B
from tests import asm_hazards as A

MFMA = "v_mfma_f32_32x32x16_bf16 a[16:31], v[0:3], v[4:7], a[16:31]"


def listing(*insts, base=0x1000):
    """objdump-style text of one function: each inst is 'mnemonic operands' or ('label', name)."""
    lines, addr = [f"{base:016x} <f>:"], base
    for ins in insts:
        if "->" in ins:  # branch: 'mnemonic -> index of the target instruction'
            mn, tgt = ins.split("->")
            lines.append(f"\t{mn.strip()} 0 // {addr:012X}: 0 <f+{0x8 * int(tgt):#x}>")
        else:
            lines.append(f"\t{ins} // {addr:012X}: 0")
        addr += 8
    return "\n".join(lines)


def problems(*insts):
    return A.check_function(A.parse(listing(*insts))["f"])


def test_valu_write_right_before_mfma_is_flagged():
    assert problems("v_accvgpr_write_b32 a16, v9", MFMA)            # accumulator element
    assert problems("v_cvt_pk_bf16_f32 v2, v8, v9", MFMA)           # A operand
    assert problems("v_mov_b32_e32 v7, v8", "s_nop 0", MFMA)         # one wait state only
    assert problems("v_accvgpr_mov_b32 a31, a40", "s_waitcnt lgkmcnt(0)", MFMA)


def test_two_wait_states_or_unrelated_writes_pass():
    assert not problems("v_accvgpr_write_b32 a16, v9", "s_nop 1", MFMA)
    assert not problems("v_mov_b32_e32 v7, v8", "s_nop 0", "s_nop 0", MFMA)
    assert not problems("v_mov_b32_e32 v8, v9", MFMA)               # not an operand
    assert not problems("v_accvgpr_write_b32 a32, v9", MFMA)        # the next tuple
    assert not problems("ds_read_b128 v[0:3], v20", MFMA)            # LDS reads: waited by counters
    assert not problems("v_cmp_gt_i32_e32 vcc, v0, v1", MFMA)        # writes no vector register


def test_paths_through_branches():
    # the MFMA heads a block entered by a branch right after a write of its accumulator
    assert problems("v_accvgpr_write_b32 a20, v9", "s_branch -> 3", "s_nop 7", MFMA)
    # the MFMA is entered only by the conditional branch at the top: the write before the
    # unconditional branch just above it is on no path into it
    assert not problems("s_cbranch_scc1 -> 4", "s_nop 1", "v_accvgpr_write_b32 a21, v9", "s_branch -> 6", MFMA,
                        "s_nop 0", "s_endpgm")
    # without that branch the write falls through into the MFMA
    assert problems("s_cbranch_scc1 -> 4", "s_nop 1", "v_accvgpr_write_b32 a21, v9", "s_nop 0", MFMA,
                    "s_nop 0", "s_endpgm")


def test_reads_of_the_result_need_twelve_wait_states():
    assert problems(MFMA, "v_accvgpr_read_b32 v40, a16")
    assert problems(MFMA, "s_nop 7", "s_nop 2", "v_accvgpr_mov_b32 a96, a31")   # 11 wait states
    assert problems(MFMA, "v_mfma_f32_32x32x16_bf16 a[32:47], v[0:3], a[16:19], a[32:47]")  # result as operand
    assert not problems(MFMA, "s_nop 7", "s_nop 3", "v_accvgpr_read_b32 v40, a16")   # 12
    assert not problems(MFMA, MFMA)                                                   # same-tuple chain
    assert not problems(MFMA, "v_accvgpr_read_b32 v40, a32")                          # another tuple
    # a loop back-edge right after the MFMA reaches a read at the loop head
    assert problems("v_accvgpr_read_b32 v40, a17", MFMA, "s_cbranch_scc1 -> 0")


@pytest.mark.skipif(not os.path.exists(B.LIB_PATH), reason="library not built")
def test_built_library_has_no_mfma_hazards():
    found, count = A.check_library(B.LIB_PATH)
    assert count > 0, "no MFMA with an AGPR destination found: the disassembly was not parsed"
    assert not found, "\n".join(f"{name}:\n  " + "\n  ".join(p[:5]) for name, p in found.items())
