"""Checks on the gfx950 code hipcc generates for the chunk kernel (CPU only).

An MFMA that reads, as its accumulator input, the result of an MFMA of a
*different* shape a few wait states after that producer was issued gave wrong
accumulators on the GPU (the compiler's hazard model accepted the distance).
The kernel source avoids such chains; this test compiles it and fails if the
generated code contains one, so a change in the source or the compiler that
reintroduces the pattern is caught before any GPU run.
"""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from gated_delta_rule_06_amd import build as kbuild

MIN_WAIT_STATES = 8


def _regs(txt):
    out = set()
    for m in re.finditer(r"\b([va])\[(\d+):(\d+)\]", txt):
        out.update(m.group(1) + str(r) for r in range(int(m.group(2)), int(m.group(3)) + 1))
    rest = re.sub(r"\b([va])\[(\d+):(\d+)\]", "", txt)
    out.update(m.group(0) for m in re.finditer(r"\b[va]\d+\b", rest))
    return out


def _kernels(asm):
    for m in re.finditer(r"^(_Z\S*kernel\S*):", asm, re.M):
        end = asm.index(".Lfunc_end", m.end())
        lines = [l.split(";")[0].strip() for l in asm[m.end():end].split("\n")]
        yield m.group(1), [l for l in lines if l and not l.startswith(".") and not l.endswith(":")]


def mixed_shape_chains(lines):
    """(producer, consumer, wait states) for every MFMA whose accumulator input
    overlaps the result of an earlier MFMA of another opcode issued fewer than
    MIN_WAIT_STATES wait states before it (straight-line order)."""
    bad = []
    for i, l in enumerate(lines):
        if not l.startswith("v_mfma"):
            continue
        op = l.split()[0]
        dst = _regs(l.split(None, 1)[1].split(",")[0])
        ws = 0
        for t in lines[i + 1:i + 40]:
            o2 = t.split()[0]
            if o2 == "s_nop":
                ws += int(t.split()[1], 0) + 1
                continue
            if ws >= MIN_WAIT_STATES:
                break
            if o2.startswith(("s_cbranch", "s_branch", "s_setpc", "s_endpgm")):
                break
            if o2.startswith("v_mfma"):
                ops = [x.strip() for x in t.split(None, 1)[1].split(",")]
                if _regs(ops[3]) & dst:
                    if o2 != op:
                        bad.append((l, t, ws))
                    break
                if _regs(ops[0]) & dst:
                    break
            ws += 1
    return bad


def test_checker_flags_the_pattern():
    lines = [
        "v_mfma_f32_16x16x32_bf16 a[0:3], v[10:13], v[14:17], a[4:7]",
        "v_add_u32_e32 v1, v2, v3",
        "v_add_u32_e32 v4, v2, v3",
        "v_mfma_f32_16x16x16_bf16 a[0:3], v[20:21], v[22:23], a[0:3]",
    ]
    assert len(mixed_shape_chains(lines)) == 1
    # same shape, or far enough apart: not flagged
    same = [lines[0], lines[1], "v_mfma_f32_16x16x32_bf16 a[0:3], v[20:23], v[24:27], a[0:3]"]
    assert mixed_shape_chains(same) == []
    far = [lines[0], "s_nop 7", "s_nop 7", lines[3]]
    assert mixed_shape_chains(far) == []


@pytest.mark.skipif(shutil.which("hipcc") is None and not os.path.exists("/opt/rocm/bin/hipcc"),
                    reason="hipcc not available")
def test_chunk_kernel_has_no_mixed_shape_accumulator_chains():
    src = os.path.join(kbuild.PKG, "csrc", "chunk.hip")
    flags = [f for f in kbuild.HIPCC_FLAGS if f not in ("-fPIC", "-shared")]
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "chunk.s")
        cmd = [kbuild.hipcc(), *flags, "--cuda-device-only", "-S", "-I",
               os.path.join(kbuild.ROOT, "include"), "-I", os.path.join(kbuild.PKG, "csrc"),
               "-o", out, src]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr[-2000:]
        asm = open(out).read()
    kernels = list(_kernels(asm))
    assert len(kernels) >= 10          # 5 configurations x (dense, varlen)
    found = {name: mixed_shape_chains(lines) for name, lines in kernels}
    found = {k: v for k, v in found.items() if v}
    assert not found, "mixed-shape MFMA accumulator chains: %r" % (found,)
