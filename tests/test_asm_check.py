"""CPU: the build-time scan for hazards around the split kernel's inline-asm
MFMAs finds a vector ALU write of an operand too close to the MFMA (also
across a branch), accepts the write once two wait states separate them, and
finds a destination that overlaps an operand."""
from tree_verify_mla_kdt_amd import asm_check

HEAD = "_Zkernel:\n"
TAIL = ".Lfunc_end0:\n"
MFMA = "\tv_mfma_f32_32x32x16_bf16 v[0:15], v[16:19], v[20:23], v[0:15]\n"


def _run(body):
    return asm_check.check(HEAD + body + TAIL)


def test_write_right_before_is_found():
    assert _run("\tv_mov_b32_e32 v21, 0\n" + MFMA)
    assert _run("\tv_accvgpr_read_b32 v17, a3\n\ts_nop 0\n" + MFMA)      # one wait state only


def test_two_wait_states_are_enough():
    assert not _run("\tv_mov_b32_e32 v21, 0\n\ts_nop 1\n" + MFMA)
    assert not _run("\tv_mov_b32_e32 v21, 0\n\tv_add_u32_e32 v40, v41, v42\n\tv_mov_b32_e32 v43, 1\n" + MFMA)
    assert not _run("\tv_mov_b32_e32 v30, 0\n" + MFMA)                     # not an operand
    assert not _run("\tds_read_b128 v[16:19], v5\n\ts_waitcnt lgkmcnt(0)\n" + MFMA)


def test_branch_predecessor_is_followed():
    body = ("\tv_mov_b32_e32 v18, 0\n\ts_cbranch_scc1 .LBB0_2\n\tv_mov_b32_e32 v40, 0\n"
            "\ts_nop 3\n.LBB0_2:\n" + MFMA)
    assert _run(body)                   # the branch path: a write, the branch, then the MFMA


def test_destination_overlapping_an_operand_is_found():
    assert _run("\ts_nop 7\n\tv_mfma_f32_32x32x16_bf16 v[0:15], v[12:15], v[20:23], v[0:15]\n")
