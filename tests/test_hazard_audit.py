"""CPU tests of the MFMA hazard audit (exact_attention_102_amd/hazard_audit.py):
the scanner on hand-written control flow, then the audit of the compiled kernels."""
import os
import shutil

import pytest

from exact_attention_102_amd import hazard_audit as ha

# The shape of the faulty code: the MFMA's block ends in a branch straight to a join block
# whose first instructions read the accumulator; the fall-through path passes through an
# exec-masked region first.
JOIN_AFTER_BRANCH = """
_Zk:
\tv_mfma_f32_32x32x16_bf16 a[48:63], v[94:97], v[4:7], a[48:63]
\ts_cbranch_vccnz .LBB0_2
; %bb.1:
\ts_and_saveexec_b64 s[0:1], s[8:9]
\tv_mov_b32_e32 v7, 0
\ts_or_b64 exec, exec, s[0:1]
.LBB0_2:
\tv_accvgpr_read_b32 v161, a63
\ts_endpgm
.Lfunc_end0:
"""


def test_scanner_finds_the_short_path_through_a_branch():
    f = ha.scan_assembly(JOIN_AFTER_BRANCH)
    assert list(f) == ["_Zk"]
    assert min(w for w, *_ in f["_Zk"]) == 1


def test_scanner_accepts_padded_paths_and_overwritten_registers():
    padded = JOIN_AFTER_BRANCH.replace("\ts_cbranch_vccnz", "\ts_nop 10\n\ts_cbranch_vccnz")
    assert ha.scan_assembly(padded) == {}
    overwritten = JOIN_AFTER_BRANCH.replace(".LBB0_2:\n", ".LBB0_2:\n\tv_accvgpr_write_b32 a63, v0\n")
    assert ha.scan_assembly(overwritten) == {}
    # an MFMA reading another MFMA's result as its A or B operand is a read too
    ab = "_Zk:\n\tv_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], v[24:27], 0\n" \
         "\tv_mfma_f32_32x32x16_bf16 v[32:47], v[0:3], v[24:27], 0\n\ts_endpgm\n.Lfunc_end0:\n"
    assert min(w for w, *_ in ha.scan_assembly(ab)["_Zk"]) == 0


def test_scanner_finds_valu_writes_read_by_an_mfma():
    """A VALU write of an MFMA operand register needs 2 wait states before the MFMA."""
    close = "_Zk:\n\tv_accvgpr_read_b32 v41, a155\n" \
            "\tv_mfma_f32_32x32x16_bf16 v[18:33], v[244:247], v[38:41], 0\n\ts_endpgm\n.Lfunc_end0:\n"
    f = ha.scan_assembly(close)
    assert min(w for w, *_ in f["_Zk"]) == 0
    assert ha.scan_assembly(close.replace("\tv_mfma", "\ts_nop 1\n\tv_mfma")) == {}
    # the C operand counts too; an unrelated register does not
    c = close.replace("v[38:41], 0", "v[0:3], v[40:55]")
    assert list(ha.scan_assembly(c)) == ["_Zk"]
    assert ha.scan_assembly(close.replace("v41, a155", "v99, a155")) == {}


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc is needed to compile the kernels' assembly")
def test_compiled_kernels_have_no_short_mfma_paths():
    res = ha.audit()
    bad = {src: sorted(funcs) for src, funcs in res.items() if funcs}
    assert not bad, bad
