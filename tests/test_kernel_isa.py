"""The decode kernel's hand-placed DPP instructions, checked in its compiled gfx950 code.

The PV step reads each probability through a DPP row broadcast inside an inline-asm
FMA, which the compiler's hazard recognizer cannot see; the kernel therefore places
an ``s_nop 1`` after the VALU write of the probability.  Hardware requires two wait
states between a VALU write of a VGPR and a DPP read of it, and a missing wait makes
the FMA read a stale value.  This test compiles the kernels to assembly with the
library's own flags and checks every DPP instruction.  It needs hipcc, not a GPU.
"""

import os
import shutil
import subprocess

import pytest

from paged_kv_cache_442_amd import build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


def compile_to_asm(tmp_path):
    out = tmp_path / "kernels.s"
    flags = [f for f in build.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc()] + flags + ["--cuda-device-only", "-S", "-I", build.INCLUDE, "-I", build.CSRC,
                                     os.path.join(build.CSRC, "kernels.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def instructions(asm):
    for line in asm.split("\n"):
        t = line.strip()
        if not t or t.startswith((";", ".")) or t.endswith(":"):
            continue
        yield t


def dpp_hazards(asm):
    """(total DPP instructions, list of (writer, reader)) with fewer than 2 wait states."""
    ins = list(instructions(asm))
    total, bad = 0, []
    for i, line in enumerate(ins):
        op = line.split()[0]
        if "_dpp" not in op:
            continue
        total += 1
        src = line.split()[2].rstrip(",")
        waits, j = 0, i - 1
        while j >= 0 and waits < 2:
            prev = ins[j].split()
            if prev[0] == "s_nop":
                waits += int(prev[1]) + 1
            elif prev[0].startswith(("s_cbranch", "s_branch")):
                break
            else:
                if prev[0].startswith("v_") and len(prev) > 1 and prev[1].rstrip(",") == src:
                    bad.append((ins[j], line))
                    break
                waits += 1
            j -= 1
    return total, bad


def test_every_dpp_read_waits_two_states_after_the_write(tmp_path):
    total, bad = dpp_hazards(compile_to_asm(tmp_path))
    assert total > 0
    assert not bad, "DPP read too soon after the VALU write: %s" % bad[:3]


def test_the_scan_catches_a_missing_wait():
    asm = "\n".join(["v_exp_f32_e32 v87, v33",
                     "v_fmac_f32_dpp v59, v87, v80 row_newbcast:0 row_mask:0xf bank_mask:0xf",
                     "v_exp_f32_e32 v88, v33",
                     "s_nop 1",
                     "v_fmac_f32_dpp v59, v88, v80 row_newbcast:0 row_mask:0xf bank_mask:0xf"])
    total, bad = dpp_hazards(asm)
    assert total == 2 and len(bad) == 1 and "v87" in bad[0][0]
