"""The compiled kernels respect the wait-state rule for their hand-written LDS
loads (CPU only: compiles the device code to gfx950 assembly and reads it).

A vector memory instruction that reads an SGPR written by a VALU instruction
needs 5 wait states in between on this GPU family.  The compiler inserts them
for the memory instructions it emits itself, but the buffer-to-LDS loads are
asm statements it cannot see into; their descriptor SGPRs (and M0) must
therefore never come from a VALU instruction fewer than 5 wait states earlier.
A violation makes a load read a stale descriptor: wrong data, or an address
outside every buffer.  An SALU write of M0 needs 1 wait state before an LDS
DMA reads it.  The scan follows every control-flow path into each load:
fall-through, branch targets and loop back-edges.
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


# Instructions after which control does not fall through to the next line.
NO_FALLTHROUGH = ("s_branch", "s_endpgm", "s_setpc_b64", "s_trap")


def is_code(x):
    return bool(x) and not x.startswith((";", "."))


def cfg(lines):
    """Predecessors of every listing line that holds an instruction: the
    previous instruction (unless it is an unconditional branch or the end of
    the program) and every branch whose target label starts the line's block.
    Labels are the lines ending in ':' that are not directives."""
    label_at, instr = {}, []
    pending = []
    for i, x in enumerate(lines):
        if x.endswith(":") and not x.startswith(";"):
            pending.append(x[:-1])
        elif is_code(x):
            for lab in pending:
                label_at[lab] = i
            pending = []
            instr.append(i)
    preds = {i: [] for i in instr}
    for a, b in zip(instr, instr[1:]):
        if not lines[a].split()[0].startswith(NO_FALLTHROUGH):
            preds[b].append(a)
    for i in instr:
        op = lines[i].split()
        if op[0].startswith(("s_branch", "s_cbranch")) and len(op) > 1 and op[1] in label_at:
            preds[label_at[op[1]]].append(i)
    return preds


def wait_states(x):
    """Wait states an instruction provides: s_nop N gives N + 1, anything else
    (conservatively) 1."""
    if x.startswith("s_nop"):
        return int(x.split()[1]) + 1
    return 1


def violations(asm_lines):
    """LDS-DMA buffer loads that can read a descriptor SGPR, the soffset SGPR or
    M0 fewer than 5 wait states after a VALU instruction wrote it, or M0 in the
    wait state right after an SALU instruction wrote it.  The look-back follows
    every control-flow predecessor (fall-through, branches, loop back-edges)."""
    lines = [x.strip() for x in asm_lines]
    preds = cfg(lines)
    found = []
    for i, line in enumerate(lines):
        if not (line.startswith("buffer_load") and line.endswith(" lds")):
            continue
        ops = [o.strip() for o in line.split(None, 1)[1].split(",")]
        read = regs(ops[1]) | {"m0"}
        if len(ops) > 2:
            read |= regs(ops[2].split()[0])
        # depth-first over paths backwards: (line, wait states so far)
        stack, seen = [(j, 0) for j in preds.get(i, [])], set()
        while stack:
            j, ws = stack.pop()
            if (j, ws) in seen or ws >= WAIT_STATES:
                continue
            seen.add((j, ws))
            x = lines[j]
            parts = x.split(None, 1)
            dst = parts[1].split(",")[0] if len(parts) > 1 else ""
            written = regs(dst)
            if parts[0].startswith("v_") and written & read:
                found.append((i, x, line))
                break
            if parts[0].startswith("s_") and "m0" in written and ws < 1:
                found.append((i, x, line))
                break
            stack.extend((k, ws + wait_states(x)) for k in preds.get(j, []))
    return found


def variant_sources(dirpath):
    """A variant of the load helpers that was tried and withdrawn: the
    descriptor's v_readfirstlane and its 5 wait states inside the descriptor
    helper's own asm statement, and no s_nop in front of the loads; written,
    with the tiled GEMM and the headers it includes, into dirpath."""
    src = open(os.path.join(build.CSRC, "lds_dma.hpp")).read()
    a = src.index("__device__ __forceinline__ i32x4 rsrc(const void *base) {")
    b = src.index("__device__ __forceinline__ uint32_t lds_addr")
    helper = (
        "__device__ __forceinline__ i32x4 rsrc(const void *base) {\n"
        "  const uint64_t a = (uint64_t)base;\n"
        "  int lo, hi;\n"
        '  asm volatile("v_readfirstlane_b32 %0, %2\\n\\tv_readfirstlane_b32 %1, %3\\n\\ts_nop 4"\n'
        '               : "=s"(lo), "=s"(hi)\n'
        '               : "v"((int)(uint32_t)a), "v"((int)(uint32_t)(a >> 32) & 0xffff));\n'
        "  i32x4 r;\n  r[0] = lo;\n  r[1] = hi;\n  r[2] = 0x7fffffff;\n  r[3] = RSRC_WORD3;\n"
        "  return r;\n}\n\n")
    variant = (src[:a] + helper + src[b:]).replace('asm volatile("s_nop 4\\n\\tbuffer_load',
                                                   'asm volatile("buffer_load')
    assert "s_nop 4\\n\\tbuffer_load" not in variant
    for name in ("gemm_tiled.hip", "device_common.hpp", "kernels.h", "tiled_geometry.hpp"):
        with open(os.path.join(dirpath, name), "w") as f:
            f.write(open(os.path.join(build.CSRC, name)).read())
    with open(os.path.join(dirpath, "lds_dma.hpp"), "w") as f:
        f.write(variant)
    return os.path.join(dirpath, "gemm_tiled.hip")


def compile_path_to_asm(path, out):
    cmd = [build.hipcc(), *build.COMMON, *build.DEVICE_FLAGS, "--offload-device-only", "-S", path,
           "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


@pytest.fixture(scope="module")
def asm_files():
    """Assembly of every kernel source, and (key "variant") of the withdrawn
    descriptor-helper variant of the tiled GEMM, compiled in parallel."""
    with tempfile.TemporaryDirectory() as tmp:
        vdir = os.path.join(tmp, "variant")
        os.makedirs(vdir)
        jobs = [(os.path.join(build.CSRC, s), os.path.join(tmp, s + ".s")) for s in KERNEL_SOURCES]
        jobs.append((variant_sources(vdir), os.path.join(tmp, "variant.s")))
        with ThreadPoolExecutor(min(8, len(jobs))) as ex:
            paths = list(ex.map(lambda j: compile_path_to_asm(*j), jobs))
        names = KERNEL_SOURCES + ["variant"]
        yield {n: open(p).read().splitlines() for n, p in zip(names, paths)}


def test_checker_finds_a_planted_violation():
    """The scan itself: a VALU write of a descriptor SGPR two instructions before
    an LDS load is caught; the same after s_nop 4 is not; a VALU write of M0, an
    SALU write of M0 right before the load, and a VALU write of the soffset
    SGPR are caught; an SALU write of M0 one wait state earlier is not."""
    bad = ["v_readfirstlane_b32 s4, v32", "v_cndmask_b32_e32 v54, v37, v28, vcc", ";;#ASMSTART",
           "buffer_load_dwordx4 v54, s[4:7], 0 offen lds"]
    assert len(violations(bad)) == 1
    good = ["v_readfirstlane_b32 s4, v32", "s_nop 4", "buffer_load_dwordx4 v54, s[4:7], 0 offen lds"]
    assert violations(good) == []
    m0 = ["v_readfirstlane_b32 m0, v3", "buffer_load_dword v1, s[8:11], 0 offen lds"]
    assert len(violations(m0)) == 1
    salu_m0 = ["s_mov_b32 m0, s2", "buffer_load_dword v1, s[8:11], 0 offen lds"]
    assert len(violations(salu_m0)) == 1
    salu_m0_ok = ["s_mov_b32 m0, s2", "s_nop 0", "buffer_load_dword v1, s[8:11], 0 offen lds"]
    assert violations(salu_m0_ok) == []
    soff = ["v_readlane_b32 s12, v40, 3", "buffer_load_dword v1, s[8:11], s12 offen lds"]
    assert len(violations(soff)) == 1


def test_checker_follows_branches_and_back_edges():
    """A hazard reached only over a branch (the write sits in another block that
    jumps to the load's block) or over a loop back-edge (the write at the end of
    the loop body, the load at its top) is caught; the straight-line
    look-back alone would miss both."""
    over_branch = [".LBB0_1:", "v_readfirstlane_b32 s4, v1", "s_branch .LBB0_3",
                   ".LBB0_2:", "s_nop 7", "s_nop 7",
                   ".LBB0_3:", "buffer_load_dwordx4 v54, s[4:7], 0 offen lds", "s_endpgm"]
    assert len(violations(over_branch)) == 1
    back_edge = ["s_nop 7", ".LBB0_1:", "buffer_load_dwordx4 v54, s[4:7], 0 offen lds",
                 "s_nop 7", "s_nop 7", "v_readfirstlane_b32 s5, v2", "s_cbranch_scc1 .LBB0_1",
                 "s_endpgm"]
    assert len(violations(back_edge)) == 1
    covered = [".LBB0_1:", "v_readfirstlane_b32 s4, v1", "s_nop 4", "s_branch .LBB0_3",
               ".LBB0_3:", "buffer_load_dwordx4 v54, s[4:7], 0 offen lds", "s_endpgm"]
    assert violations(covered) == []


@pytest.mark.parametrize("src", KERNEL_SOURCES)
def test_no_valu_sgpr_hazard_before_lds_loads(asm_files, src):
    found = violations(asm_files[src])
    assert not found, f"{src}: {found[:3]}"


def test_scan_catches_the_descriptor_helper_variant(asm_files):
    """The withdrawn variant (see variant_sources), rebuilt from the current
    helpers and compiled with the tiled GEMM, has the descriptor covered but
    leaves M0 exposed: the compiler sets M0 for each load with an SALU
    instruction (s_mov_b32, or s_cselect_b32 choosing the LDS address or -1)
    right before it, with no wait state, so the load may use the previous M0 -
    another stage's LDS address, or -1 - for its whole 1 KiB.  The scan finds
    exactly that hazard there, and none in the current helpers."""
    found = violations(asm_files["variant"])
    assert found
    for _, writer, _ in found:
        op, dst = writer.split(None, 1)
        assert op.startswith("s_") and dst.split(",")[0].strip() == "m0", writer
