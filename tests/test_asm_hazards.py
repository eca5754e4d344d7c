"""The kernels that issue MFMAs as inline assembly (fa_fwd_d128.hip,
fa_fwd_short.hip) place the wait states gfx950 requires by hand.  This
compiles them for gfx950 (no GPU needed) and scans the generated code of
every instantiation, so that a register-allocation change that adds a copy
next to an MFMA is caught before it runs."""

import os
import shutil
import subprocess
import tempfile

import pytest

from asm_hazards import findings, scan
from exact_attention_25_amd import build_lib

HIPCC = build_lib.HIPCC


def test_scanner_flags_planted_hazards():
    clean = ["s_nop 1", "v_mfma_f32_32x32x16_f16 v[0:15], v[16:19], a[0:3], v[0:15]", "s_nop 7", "s_nop 7",
             "v_add_f32_e32 v20, v0, v1"]
    assert findings(clean) == []
    write_then_mfma = ["v_mov_b32_e32 v19, v30", "v_mfma_f32_32x32x16_f16 v[0:15], v[16:19], a[0:3], v[0:15]"]
    assert len(findings(write_then_mfma)) == 1
    one_state = ["v_mov_b32_e32 v19, v30", "s_nop 0", "v_mfma_f32_32x32x16_f16 v[0:15], v[16:19], a[0:3], v[0:15]"]
    assert len(findings(one_state)) == 1
    agpr_copy = ["v_accvgpr_read_b32 v35, a111", "v_mfma_f32_32x32x16_bf16 v[0:15], v[32:35], a[80:83], v[0:15]"]
    assert len(findings(agpr_copy)) == 1
    read_early = ["v_mfma_f32_32x32x16_f16 v[0:15], v[16:19], a[0:3], 0", "s_nop 7",
                  "v_max_f32_e32 v40, v3, v40"]
    assert len(findings(read_early)) == 1
    agpr_read_early = ["v_mfma_f32_32x32x16_f16 a[0:15], v[16:19], v[20:23], a[0:15]",
                       "v_accvgpr_read_b32 v1, a4"]
    assert len(findings(agpr_read_early)) == 1


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("source", ["fa_fwd_d128.hip", "fa_fwd_short.hip"])
def test_inline_asm_kernels_have_no_mfma_hazards(source):
    flags = [f for f in build_lib.hipcc_flags() if f not in ("-shared", "-fPIC")]
    with tempfile.TemporaryDirectory(prefix="fa_asm_") as d:
        out = os.path.join(d, source + ".s")
        cmd = [HIPCC] + flags + ["--cuda-device-only", "-S", os.path.join(build_lib.CSRC, source), "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        result = scan(open(out).read())
    kernels = {k: v for k, v in result.items() if "kernel" in k}
    assert kernels, "no kernels found in the assembly of " + source
    bad = {k: v for k, v in kernels.items() if v}
    assert not bad, "\n".join("%s: %s" % (k, "; ".join(v[:3])) for k, v in bad.items())
