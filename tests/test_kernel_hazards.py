"""The compiled kernels respect the wait-state rule for their hand-written LDS
loads (CPU only: compiles the device code to gfx950 assembly and reads it).

A vector memory instruction that reads an SGPR written by a VALU instruction
needs 5 wait states in between on this GPU family.  The compiler inserts them
for the memory instructions it emits itself, but the buffer-to-LDS loads are
asm statements it cannot see into; their descriptor SGPRs (and M0) must
therefore never come from a VALU instruction fewer than 5 wait states earlier.
A violation makes a load read a stale descriptor: wrong data, or an address
outside every buffer.
"""
import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from megatron_tensor_mlp_amd import build

KERNEL_SOURCES = [s for s in build.SOURCES if s.endswith(".hip")]
WAIT_STATES = 5


def regs(tok):
    """SGPRs (and M0) an operand names."""
    tok = tok.strip()
    if tok == "m0":
        return {"m0"}
    m = re.match(r"s\[(\d+):(\d+)\]$", tok)
    if m:
        return {f"s{i}" for i in range(int(m.group(1)), int(m.group(2)) + 1)}
    m = re.match(r"s(\d+)$", tok)
    return {tok} if m else set()


def violations(asm_lines):
    """LDS-DMA buffer loads whose descriptor SGPRs or M0 a VALU instruction wrote
    fewer than WAIT_STATES wait states before (look-back over the preceding
    lines of the listing)."""
    lines = [x.strip() for x in asm_lines]
    found = []
    for i, line in enumerate(lines):
        if not (line.startswith("buffer_load") and line.endswith(" lds")):
            continue
        ops = line.split(None, 1)[1].split(",")
        read = regs(ops[1]) | {"m0"}
        ws, j = 0, i - 1
        while j >= 0 and ws < WAIT_STATES:
            x = lines[j]
            j -= 1
            if not x or x.startswith(";") or x.startswith("."):
                continue  # comments, directives and labels (the look-back runs on
                # through block starts: conservative for code laid out in order)
            if x.startswith("s_nop"):
                ws += int(x.split()[1]) + 1
                continue
            parts = x.split(None, 1)
            dst = parts[1].split(",")[0] if len(parts) > 1 else ""
            if parts[0].startswith("v_") and regs(dst) & read:
                found.append((i, x, line))
                break
            ws += 1
    return found


def compile_to_asm(src, outdir):
    out = os.path.join(outdir, src + ".s")
    cmd = [build.hipcc(), *build.COMMON, *build.DEVICE_FLAGS, "--offload-device-only", "-S",
           os.path.join(build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def asm_files():
    with tempfile.TemporaryDirectory() as tmp:
        with ThreadPoolExecutor(min(8, len(KERNEL_SOURCES))) as ex:
            paths = list(ex.map(lambda s: compile_to_asm(s, tmp), KERNEL_SOURCES))
        yield {s: open(p).read().splitlines() for s, p in zip(KERNEL_SOURCES, paths)}


def test_checker_finds_a_planted_violation():
    """The scan itself: a VALU write of a descriptor SGPR two instructions before
    an LDS load is caught; the same after s_nop 4 is not."""
    bad = ["v_readfirstlane_b32 s4, v32", "v_cndmask_b32_e32 v54, v37, v28, vcc", ";;#ASMSTART",
           "buffer_load_dwordx4 v54, s[4:7], 0 offen lds"]
    assert len(violations(bad)) == 1
    good = ["v_readfirstlane_b32 s4, v32", "s_nop 4", "buffer_load_dwordx4 v54, s[4:7], 0 offen lds"]
    assert violations(good) == []
    m0 = ["v_readfirstlane_b32 m0, v3", "buffer_load_dword v1, s[8:11], 0 offen lds"]
    assert len(violations(m0)) == 1


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_valu_sgpr_hazard_before_lds_loads(asm_files, src):
    found = violations(asm_files[src])
    assert not found, f"{src}: {found[:3]}"
