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

3. No kernel keeps values in the accumulation registers (AGPRs), and no instruction reads
an MFMA result before the MFMA has written it.  A read of an MFMA's destination needs
independent instructions after the MFMA (8 wait states for the 16x16x32 forms, 12 for
32x32x16: what the compiler itself pads a straight-line read with, checked below), and
nothing in hardware enforces it: a read too soon returns the register's old value.  The
one build that used AGPRs (the decode kernel for groups of 8 compiled for three
workgroups per CU) read its QK accumulator with v_accvgpr_read three wait states after
the last MFMA, on the branch that skips the claim of the next unit, so the scores came
from the previous tile; it gave wrong outputs at g = 8 on the GPU.  The scan below walks
every path from each MFMA (branches included) and finds that read in that build; it
finds none in the kernels as built.

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


# --------------------------------------------------------------------------- MFMA results
# Wait states a read of an MFMA's destination must trail the MFMA by.
MFMA_READ_WAITS = {"v_mfma_f32_16x16x32_bf16": 8, "v_mfma_f32_16x16x32_f16": 8,
                   "v_mfma_f32_32x32x16_bf16": 12, "v_mfma_f32_32x32x16_f16": 12}
_BRANCH = re.compile(r"^s_c?branch")
_STORES = ("global_store", "buffer_store", "ds_write", "ds_store", "flat_store", "scratch_store")


def vector_regs(tok):
    """{(bank, index)} of a VGPR / AGPR operand such as v5, v[2:5], a3, a[0:3]."""
    tok = tok.rstrip(",")
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def code_with_labels(body):
    """(instructions, {label: index of the instruction after it}) of one kernel."""
    ins, labels = [], {}
    for line in body.split("\n"):
        s = line.split(";")[0].strip()
        if not s:
            continue
        if s.endswith(":"):
            if s.startswith("."):
                labels[s[:-1]] = len(ins)
            continue
        if not s.startswith("."):
            ins.append(s)
    return ins, labels


def _reads(op, operands):
    regs = operands if op.startswith(_STORES) else operands[1:]
    return set().union(*[vector_regs(x) for x in regs]) if regs else set()


def _writes(op, operands):
    if op.startswith(_STORES) or op.startswith("s_") or not operands:
        return set()
    return vector_regs(operands[0])


def mfma_read_hazards(body):
    """[(mfma, reader, wait states)] for every path (fall-through and branch targets) on
    which a non-MFMA instruction reads an MFMA's destination too soon.  A register
    rewritten on the way no longer counts; MFMA-to-MFMA accumulation chains are left
    to the hardware."""
    ins, labels = code_with_labels(body)
    bad = []
    for i, line in enumerate(ins):
        parts = line.split()
        if parts[0] not in MFMA_READ_WAITS:
            continue
        need = MFMA_READ_WAITS[parts[0]]
        seen = {}
        stack = [(i + 1, 0, frozenset(vector_regs(parts[1])))]
        while stack:
            j, waits, live = stack.pop()
            while j < len(ins) and waits < need and live:
                if seen.get((j, live), 1 << 30) <= waits:
                    break
                seen[(j, live)] = waits
                toks = ins[j].split()
                op = toks[0]
                if not op.startswith("v_mfma") and _reads(op, toks[1:]) & live:
                    bad.append((line, ins[j], waits))
                    break
                live = live - _writes(op, toks[1:])
                if op == "s_endpgm":
                    break
                waits += int(toks[1], 0) + 1 if op == "s_nop" else 1
                if _BRANCH.match(op):
                    if toks[1] in labels:
                        stack.append((labels[toks[1]], waits, live))
                    if op == "s_branch":
                        break
                j += 1
    return bad


def test_no_mfma_result_is_read_too_soon(asm, prefill_asm):
    checked = 0
    for text in (asm, prefill_asm):
        for name, body in kernel_bodies(text, r".").items():
            if "v_mfma" in body:
                checked += 1
                assert not mfma_read_hazards(body), (name, mfma_read_hazards(body)[:2])
    assert checked >= 14  # 6 decode kernels on MFMA, 8 prefill kernels


def test_mfma_read_waits_match_the_compilers_own_padding(tmp_path):
    """The compiler pads a straight-line read of each MFMA form with exactly these waits."""
    src = tmp_path / "mfma_read.hip"
    forms = {"v_mfma_f32_16x16x32_bf16": ("4", "__bf16", "mfma_f32_16x16x32_bf16", 3),
             "v_mfma_f32_16x16x32_f16": ("4", "_Float16", "mfma_f32_16x16x32_f16", 3),
             "v_mfma_f32_32x32x16_bf16": ("16", "__bf16", "mfma_f32_32x32x16_bf16", 15),
             "v_mfma_f32_32x32x16_f16": ("16", "_Float16", "mfma_f32_32x32x16_f16", 15)}
    code = ["#include <hip/hip_runtime.h>"]
    for k, (n, t, b, last) in enumerate(forms.values()):
        code.append(
            "__global__ void k%d(const %s* a, const %s* b, float* o) {"
            " typedef %s x8 __attribute__((ext_vector_type(8)));"
            " typedef float acc __attribute__((ext_vector_type(%s)));"
            " acc c = {}; c = __builtin_amdgcn_%s(((const x8*)a)[threadIdx.x], ((const x8*)b)[threadIdx.x], c, 0, 0, 0);"
            " o[threadIdx.x] = c[0] * 3.0f + c[%d]; }" % (k, t, t, t, n, b, last))
    src.write_text("\n".join(code))
    out = tmp_path / "mfma_read.s"
    res = subprocess.run([build.hipcc(), "--offload-arch=gfx950", "-O3", "--cuda-device-only", "-S",
                          str(src), "-o", str(out)], capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    found = {}
    for body in kernel_bodies(out.read_text(), r".").values():
        ins, _ = code_with_labels(body)
        at = next(i for i, x in enumerate(ins) if x.startswith("v_mfma"))
        waits, j = 0, at + 1
        while not _reads(ins[j].split()[0], ins[j].split()[1:]) & vector_regs(ins[at].split()[1]):
            waits += int(ins[j].split()[1], 0) + 1 if ins[j].startswith("s_nop") else 1
            j += 1
        found[ins[at].split()[0]] = waits
    assert found == MFMA_READ_WAITS


def test_the_mfma_scan_finds_the_read_of_the_agpr_build(tmp_path):
    """The decode kernel for groups of 8 built for three workgroups per CU (the 16-bit
    ones put their QK accumulators in AGPRs): the scan finds the too-early v_accvgpr_read,
    in g = 8 kernels only."""
    src = open(os.path.join(build.CSRC, "kernels.hip")).read()
    kept = "(GW >= 4 ? 2 : 4);"
    assert src.count(kept) == 1
    variant = tmp_path / "kernels.hip"
    variant.write_text(src.replace(kept, "(GW == 8 ? 3 : GW >= 4 ? 2 : 4);"))
    out = tmp_path / "variant.s"
    flags = [f for f in build.HIP_FLAGS if f not in ("-shared", "-fPIC")]
    res = subprocess.run([build.hipcc()] + flags + ["--cuda-device-only", "-S", "-I", build.INCLUDE,
                                                    "-I", build.CSRC, str(variant), "-o", str(out)],
                         capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    flagged = {}
    for name, body in kernel_bodies(out.read_text(), r"decode_partition_kernel").items():
        flagged[name] = mfma_read_hazards(body)
    hit = {n for n, h in flagged.items() if h}
    assert hit and all("Li8ELi1E" in n for n in hit), sorted(hit)
    assert all(r.startswith("v_accvgpr_read") and w < 8 for n in hit for _, r, w in flagged[n])


def test_the_mfma_scan_follows_branches():
    body = "\n".join(["v_mfma_f32_16x16x32_bf16 v[2:5], v[6:9], v[10:13], 0",
                      "s_cbranch_scc1 .LBB0_2",
                      "s_nop 7",
                      "v_add_f32_e32 v1, v2, v3",
                      ".LBB0_2:",
                      "v_mov_b32_e32 v2, 0",
                      "v_add_f32_e32 v1, v3, v4",
                      "v_add_f32_e32 v1, v5, v4"])
    bad = mfma_read_hazards(body)
    # Via the branch: v2 is rewritten before any read, v3 is read 2 wait states after
    # (the branch and the move); the fall-through path waits 9 states.
    assert [(r, w) for _, r, w in bad] == [("v_add_f32_e32 v1, v3, v4", 2)]
