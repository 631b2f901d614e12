"""The built gfx950 code never reads an MFMA result too early (see
log_linear_attention_attn_amd/isa_check.py).  CPU only: compiles to assembly."""
import shutil

import pytest

from log_linear_attention_attn_amd import isa_check


@pytest.mark.skipif(shutil.which("hipcc") is None and not __import__("os").path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_no_early_mfma_result_reads():
    bad = isa_check.scan(isa_check.device_asm())
    assert not bad, "\n".join(bad[:10])


def test_scanner_flags_a_branch_after_mfma():
    asm = """_Zfake:
\tv_mfma_f32_16x16x32_bf16 a[0:3], v[6:9], v[78:81], a[0:3]
\ts_cbranch_scc1 .LBB0_2
\ts_nop 7
\ts_nop 7
.LBB0_2:
\tv_accvgpr_read_b32 v5, a3
\ts_endpgm
"""
    assert len(isa_check.scan(asm)) == 1
    ok = asm.replace("\ts_cbranch_scc1 .LBB0_2\n", "")
    assert isa_check.scan(ok) == []
