"""The decode kernel's gfx950 assembly (built here, on the CPU): nothing may
read or write a score-MFMA chain's accumulator while the matrix core is still
writing it.  The score MFMAs are inline asm, which the compiler's hazard
recognizer cannot see, so this is checked on the instruction stream."""
import shutil

import pytest

from layout_agnostic_latent_amd import asm_check, build


def test_scan_flags_a_copy_of_an_in_flight_accumulator():
    # the pattern a register-allocator split would produce: a copy between
    # two chained MFMAs reads the first one's result before it is written
    bad_asm = """
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[2:17], v[20:23], v[30:33], v[2:17]
\t;;#ASMEND
\tv_mov_b64_e32 v[40:41], v[2:3]
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[40:55], v[24:27], v[30:33], v[40:55]
\ts_nop 7
\ts_nop 7
\ts_nop 3
\t;;#ASMEND
\tv_add_f32_e32 v60, v40, v41
"""
    assert len(asm_check.scan(bad_asm)) == 1


def test_scan_accepts_a_chain_and_its_guarded_end():
    good_asm = """
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[2:17], v[20:23], v[30:33], 0
\t;;#ASMEND
\tds_read_b128 v[20:23], v100
\tv_exp_f32_e32 v60, v61
\t;;#ASMSTART
\tv_mfma_f32_32x32x16_bf16 v[2:17], v[24:27], v[30:33], v[2:17]
\ts_nop 7
\ts_nop 7
\ts_nop 3
\t;;#ASMEND
\tv_max3_f32 v60, v2, v3, v4
"""
    assert asm_check.scan(good_asm) == []
    # without the trailing wait states the first read of the result is flagged
    assert len(asm_check.scan(good_asm.replace("\ts_nop 7\n\ts_nop 7\n\ts_nop 3\n", ""))) == 1


def test_scan_counts_independent_instructions_as_wait_states():
    # the chain's wait states filled with other work: 20 independent
    # instructions (among them MFMAs into other accumulators) before the read
    body = "".join(f"\tv_mfma_f32_32x32x16_bf16 a[{16 * k}:{16 * k + 15}], v[44:47], v[48:51], a[{16 * k}:{16 * k + 15}]\n"
                   f"\tds_read_b64_tr_b16 v[52:53], v100\n\ts_waitcnt lgkmcnt(2)\n\tds_read_b64_tr_b16 v[54:55], v101\n"
                   for k in range(5))
    asm = ("\t;;#ASMSTART\n\tv_mfma_f32_32x32x16_bf16 v[18:33], v[36:39], v[40:43], v[18:33]\n\t;;#ASMEND\n"
           + body + "\tv_max3_f32 v60, v18, v19, v20\n")
    assert asm_check.scan(asm) == []
    # one step fewer leaves only 16 wait states
    short = asm.replace(body, body[:body.rindex("\tv_mfma")])
    assert len(asm_check.scan(short)) == 1
    # a label or a branch inside the window is reported
    assert len(asm_check.scan(asm.replace("\tds_read_b64_tr_b16 v[52:53], v100\n", ".LBB0_7:\n", 1))) == 1
    assert len(asm_check.scan(asm.replace("\ts_waitcnt lgkmcnt(2)\n", "\ts_cbranch_scc1 .LBB0_9\n", 1))) == 1


@pytest.mark.skipif(shutil.which(build.hipcc()) is None and not __import__("os").path.exists(build.hipcc()),
                    reason="hipcc not available")
def test_decode_kernel_never_touches_an_in_flight_score_accumulator():
    text = asm_check.compile_asm()
    chain = [l for l in text.split("\n") if "v_mfma" in l and ("v[2:17]" in l or "v[18:33]" in l)]
    assert len(chain) > 100, "score-chain MFMAs not found in the assembly"
    assert asm_check.scan(text) == []
