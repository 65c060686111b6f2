"""Register placement of the fp6 packing instruction in the built quantizer.

V_CVT_SCALEF32_2XPK16_FP6_F32 (the W4A4 quantizer's code packing, ``quant_act.hip``)
gave one wrong dword per lane on gfx950 when its result registers overlapped
its second source, and the register allocator is free to choose such a
placement under pressure (one instance did, and the codes it packed were wrong
at odd K positions).  The kernel therefore issues the instruction with an
early-clobber result.  This compiles ``quant_act.hip`` for gfx950 with the
library's own flags (device code only, no GPU needed) and checks every packing
instruction of every instance: the result registers share none with either
source."""

import os
import re
import subprocess
import tempfile

import pytest

from bit_ptq_looped_amd import build as B

PACK = re.compile(r"v_cvt_scalef32_2xpk16_fp6_f32\s+v\[(\d+):(\d+)\],\s*v\[(\d+):(\d+)\],\s*v\[(\d+):(\d+)\]")


def regs(lo, hi):
    return set(range(int(lo), int(hi) + 1))


@pytest.mark.timeout(600)
def test_pack_result_never_overlaps_its_sources():
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    src = os.path.join(B.CSRC, "quant_act.hip")
    flags = [f for f in B.COMMON if f not in ("-fPIC", "-Wall", "-Wno-unused-function")]
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "quant_act.s")
        r = subprocess.run([hipcc, *flags, f"-I{B.CSRC}", "--cuda-device-only", "-S", src, "-o", out],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        text = open(out).read()
    found = PACK.findall(text)
    assert len(found) >= 8, "expected the packing instruction in every fp6 instance"
    for m in found:
        dst, s0, s1 = regs(m[0], m[1]), regs(m[2], m[3]), regs(m[4], m[5])
        assert len(dst) == 6 and len(s0) == 16 and len(s1) == 16
        assert not (dst & s0) and not (dst & s1), f"result v[{m[0]}:{m[1]}] overlaps a source: {m}"
