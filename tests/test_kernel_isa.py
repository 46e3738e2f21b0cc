"""Properties of the kernels' compiled gfx950 code that the compiler does not guarantee.

1. The PV step reads each probability through a DPP row broadcast inside an inline-asm
FMA, which the compiler's hazard recognizer cannot see; the kernel therefore places
an ``s_nop 1`` after the VALU write of the probability.  Hardware requires two wait
states between a VALU write of a VGPR and a DPP read of it, and a missing wait makes
the FMA read a stale value.  Every DPP instruction is checked.

2. A lane's V chunk of 8 fp16 values sits in 4 dwords, and each must be widened on its
own.  A bit cast of a vector element taken as an lvalue once made the compiler widen
element 0 four times.  A 16-token tile is 4 wave-wide loads of 4 rows, so the fp16
kernels must convert from 4 x 4 = 16 distinct registers (the faulty code used 4).

3. No kernel keeps values in the accumulation registers (AGPRs).  The one build that did
(the decode kernel for groups of 8 compiled for three workgroups per CU, which moved the
MFMA accumulators there) gave wrong outputs at g = 8 on the GPU, and no cause was found
in its code; the kernels stay in VGPRs.

4. No kernel uses scratch (private) memory.  A lane-dependent choice between two members
of one small object (the prefill kernel's two block bases of a tile) once became a
lane-dependent address into a private array: scratch loads inside the tile loop, whose
wait also held up the tile's K/V loads.

The kernels are compiled to assembly with the library's own flags; hipcc is needed,
not a GPU.
"""

import re

import os
import shutil
import subprocess

import pytest

from paged_kv_cache_442_amd import build

pytestmark = pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    return compile_to_asm(tmp_path_factory.mktemp("isa"))


@pytest.fixture(scope="module")
def prefill_asm(tmp_path_factory):
    return compile_to_asm(tmp_path_factory.mktemp("isa_prefill"), "prefill.hip")


def compile_to_asm(tmp_path, source="kernels.hip"):
    out = tmp_path / (source + ".s")
    flags = [f for f in build.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [build.hipcc()] + flags + ["--cuda-device-only", "-S", "-I", build.INCLUDE, "-I", build.CSRC,
                                     os.path.join(build.CSRC, source), "-o", str(out)]
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


def test_every_dpp_read_waits_two_states_after_the_write(asm):
    total, bad = dpp_hazards(asm)
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


def kernel_bodies(asm, pattern):
    """{symbol: text} of the kernels whose symbol matches ``pattern``."""
    starts = [(m.start(), m.group(1)) for m in re.finditer(r"^(_Z\S+):", asm, re.M)]
    out = {}
    for i, (pos, name) in enumerate(starts):
        if re.search(pattern, name):
            end = starts[i + 1][0] if i + 1 < len(starts) else len(asm)
            out[name] = asm[pos:end]
    return out


def f16_widen_sources(body):
    return {line.split()[2].rstrip(",") for line in instructions(body)
            if line.split()[0].startswith("v_cvt_f32_f16")}


def test_fp16_decode_widens_every_dword_of_a_chunk(asm):
    kernels = kernel_bodies(asm, r"decode_partition_kernel.*ElemF16")
    assert len(kernels) == 4
    for name, body in kernels.items():
        assert len(f16_widen_sources(body)) >= 16, name


def test_the_widen_scan_catches_one_dword_widened_four_times():
    body = "\n".join(["v_cvt_f32_f16_sdwa v73, v30 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:WORD_1",
                      "v_cvt_f32_f16_e32 v74, v30"] * 4)
    assert f16_widen_sources(body) == {"v30"}


def agpr_use(asm):
    """(largest .agpr_count in the kernel metadata, number of AGPR copy instructions)."""
    counts = [int(c) for c in re.findall(r"\.agpr_count:\s+(\d+)", asm)]
    copies = sum(1 for line in instructions(asm) if line.split()[0].startswith("v_accvgpr"))
    return (max(counts) if counts else 0), copies, len(counts)


def test_no_kernel_uses_agprs(asm, prefill_asm):
    for text in (asm, prefill_asm):
        most, copies, n = agpr_use(text)
        assert n > 0
        assert most == 0 and copies == 0, (most, copies)


def test_the_agpr_scan_sees_an_accumulator_copy():
    text = "\n".join(["  - .agpr_count:     4", "v_accvgpr_read_b32 v21, a3"])
    assert agpr_use(text) == (4, 1, 1)


def scratch_use(asm):
    """(largest private segment of any kernel, scratch instructions, kernels seen)."""
    sizes = [int(m) for m in re.findall(r"\.private_segment_fixed_size:\s+(\d+)", asm)]
    insts = sum(1 for t in instructions(asm) if t.startswith("scratch_"))
    return (max(sizes) if sizes else 0), insts, len(sizes)


def test_no_kernel_uses_scratch(asm, prefill_asm):
    for text in (asm, prefill_asm):
        most, insts, n = scratch_use(text)
        assert n > 0
        assert most == 0 and insts == 0, (most, insts)


def test_the_scratch_scan_sees_a_spill():
    text = "\n".join(["    .private_segment_fixed_size: 16", "scratch_load_dwordx2 v[80:81], v182, off"])
    assert scratch_use(text) == (16, 1, 1)
