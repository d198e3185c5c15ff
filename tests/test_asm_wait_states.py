"""Wait states between the matrix cores and inline assembly (CPU only).

On CDNA a VALU, LDS or memory instruction that reads the result registers of
an MFMA must issue a number of wait states after it (up to 19 for a 16-pass
MFMA); the compiler inserts them (s_nop) for the instructions it generates,
but not for inline assembly.  Several kernels feed MFMA results to inline asm
(v_max3_f32 / v_max_f32 in the softmax).  This test compiles every kernel
source for gfx950 with the library's flags, finds each inline-asm instruction
whose VGPR operands (any operand of an LDS or memory instruction, the sources
of a VALU one) an MFMA wrote, and checks that at least 19 wait states (one per
instruction, n + 1 per s_nop n) separate them along the straight-line code
before it (the scan stops at an unconditional branch).  A planted asm store of
MFMA results right after the MFMA (the mistake this guards against) is caught.
"""

import os
import re
import shutil
import subprocess
import tempfile

import pytest

from transformer_attention_sdpa_amd import build_lib

NEEDED = 19  # 16-pass XDL write of a VGPR, then a non-MFMA read of it

pytestmark = pytest.mark.skipif(not shutil.which(build_lib.HIPCC) and not os.path.exists(build_lib.HIPCC),
                                reason="hipcc not available")


def _device_asm(src, out):
    flags = [f for f in build_lib.FLAGS if f not in ("-fPIC",)]
    subprocess.run([build_lib.HIPCC, *flags, "-S", "--cuda-device-only", os.path.join(build_lib.CSRC, src),
                    "-o", out], check=True, capture_output=True)
    return open(out).read().split("\n")


def _regs(operands):
    """VGPR numbers named by an operand list (v7, v[4:7])."""
    regs = set()
    for a, b in re.findall(r"v\[(\d+):(\d+)\]", operands):
        regs.update(range(int(a), int(b) + 1))
    for a in re.findall(r"(?<![\w\[:])v(\d+)\b", operands):
        regs.add(int(a))
    return regs


def _violations(lines):
    bad = []
    for i, line in enumerate(lines):
        if i == 0 or "ASMSTART" not in lines[i - 1]:
            continue
        m = re.match(r"\s*(v_\w+|ds_\w+|global_\w+|buffer_\w+)\s+(.*)", line)
        if not m:
            continue
        ops = m.group(2).split(",")
        # the first operand of a VALU op is its destination; DS/memory ops read all of theirs
        reads = _regs(",".join(ops[1:] if m.group(1).startswith("v_") else ops))
        ws = 0
        for j in range(i - 1, max(0, i - 400), -1):
            t = lines[j].strip()
            if not t or t.startswith((";", ".")):
                continue
            if t.startswith(("s_branch", "s_endpgm", "s_setpc")):
                break  # the code above does not fall through to this point
            mm = re.match(r"v_mfma\S*\s+(v\[\d+:\d+\])", t)
            if mm:
                if _regs(mm.group(1)) & reads and ws < NEEDED:
                    bad.append((i, ws, t, line.strip()))
                if _regs(mm.group(1)) & reads:
                    break
            ns = re.match(r"s_nop\s+(\d+)", t)
            ws += int(ns.group(1)) + 1 if ns else 1
            if ws >= NEEDED:
                break
    return bad


@pytest.mark.parametrize("src", [s for s in build_lib.SOURCES if s.endswith(".hip")])
def test_inline_asm_reads_mfma_results_after_enough_wait_states(src):
    with tempfile.TemporaryDirectory() as d:
        lines = _device_asm(src, os.path.join(d, "k.s"))
    bad = _violations(lines)
    assert not bad, "\n".join(f"line {i}: {ws} wait states after `{t}` before `{u}`" for i, ws, t, u in bad[:5])
