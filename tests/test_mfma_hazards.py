"""Host check of the compiled MFMA kernels: no MFMA result is used sooner after a taken branch than
the compiler allows on straight-line code.

An MFMA writes its result several cycles after it issues, and the hardware does not hold back a
VALU instruction (an accumulator copy included) that reads or writes that result early: the
compiler separates the two by wait states.  On straight-line code it always does; across a taken
branch it once did not (an accumulator copied out at the join of a branch that skipped a block,
two instructions after the chain's last MFMA), and the copy then read the value of the previous
product on some builds.  This test compiles the kernels to gfx950 assembly and, from every MFMA,
follows the fall-through and taken-branch paths to the first instruction that uses its result
registers (other than a dependent MFMA taking them as its accumulator, which the hardware orders).
Each opcode's required distance is taken from the compiler's own choice on paths without a taken
branch (the smallest distance it leaves there); a path through a taken branch that is shorter
fails.  A path on which the execution mask is known to be zero (an s_cbranch_execz taken, or an
s_cbranch_execnz not taken, and no write of exec since) runs VALU instructions on no lanes, so
those are not uses there; instructions that ignore the mask (MFMA, v_readlane, v_readfirstlane,
v_writelane) still are.  No GPU is needed.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile
from concurrent.futures import ThreadPoolExecutor

import pytest

from state_space_sequence_m3_amd import build as m3build

SOURCES = ("backward.hip", "prefill.hip")   # the translation units with MFMA kernels
WINDOW = 24                                 # wait states followed from each MFMA


def _assembly(src: str, out_dir: str) -> str:
    out = os.path.join(out_dir, src + ".s")
    flags = [f for f in m3build.compile_flags() if f != "-Wall"]
    cmd = [m3build.hipcc()] + flags + ["--cuda-device-only", "-S", os.path.join(m3build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out


def _regs(tok: str):
    m = re.match(r"([av])\[(\d+):(\d+)\]$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"([av])(\d+)$", tok)
    return {(m.group(1), int(m.group(2)))} if m else set()


def _split_kernels(path: str):
    """Kernels of an assembly file, one per function symbol."""
    out = []
    with open(path) as f:
        text = f.read().split("\n")
    starts = [i for i, l in enumerate(text) if re.match(r"^_Z\S*:", l)]
    for a, b in zip(starts, starts[1:] + [len(text)]):
        name = text[a].split(":")[0]
        ins, labels = [], {}
        for raw in text[a + 1:b]:
            line = raw.split(";")[0].strip()
            if not line or line.startswith("."):
                if line.endswith(":") and line.startswith("."):
                    labels[line[:-1]] = len(ins)
                continue
            if line.endswith(":"):
                labels[line[:-1]] = len(ins)
                continue
            op = line.split()[0]
            ops = [o.strip() for o in line[len(op):].split(",")] if len(line) > len(op) else []
            ins.append((op, ops))
        out.append((name, ins, labels))
    return out


def _use(op, ops, dst):
    """How instruction (op, ops) touches the result registers `dst` of an earlier MFMA: "use"
    (reads or writes them), "chain" (an MFMA accumulating onto them: the hardware orders it, and
    later readers see its result, which is followed from there), or None."""
    if op.startswith("v_mfma") and len(ops) >= 4:
        if dst & (_regs(ops[1]) | _regs(ops[2])):
            return "use"
        if dst & _regs(ops[3]):
            return "chain"
        return "use" if dst & _regs(ops[0]) else None
    for o in ops:
        if dst & _regs(o):
            return "use"
    return None


_EXEC_FREE = ("v_mfma", "v_readlane", "v_readfirstlane", "v_writelane")   # run whatever exec holds


def _writes_exec(op, ops):
    return "saveexec" in op or (op.startswith("s_") and bool(ops) and ops[0] == "exec")


def _distances(ins, labels):
    """(mfma opcode, distance, through a taken branch) for each MFMA and each path to a use."""
    found = []
    for i, (op, ops) in enumerate(ins):
        if not op.startswith("v_mfma"):
            continue
        dst = _regs(ops[0])
        stack = [(i + 1, 0, False, False, frozenset())]
        while stack:
            k, dist, taken, exec_zero, seen = stack.pop()
            while k < len(ins) and dist < WINDOW:
                o, oo = ins[k]
                if o == "s_endpgm":
                    break
                if o.startswith("s_nop"):
                    dist += int(oo[0], 0) + 1
                    k += 1
                    continue
                u = _use(o, oo, dst)
                if u == "use" and exec_zero and not o.startswith(_EXEC_FREE):
                    u = None   # no lane runs it
                if u == "use":
                    found.append((op, dist, taken))
                if u is not None:
                    break
                if _writes_exec(o, oo):
                    exec_zero = False
                if o.startswith("s_cbranch") or o == "s_branch":
                    tgt = labels.get(oo[0]) if oo else None
                    if tgt is not None and (k, tgt) not in seen:
                        stack.append((tgt, dist + 1, True, exec_zero or o == "s_cbranch_execz",
                                      seen | {(k, tgt)}))
                    if o == "s_branch":
                        break
                    if o == "s_cbranch_execnz":
                        exec_zero = True   # falling through: exec is zero
                dist += 1
                k += 1
    return found


@pytest.fixture(scope="module")
def assembly():
    with tempfile.TemporaryDirectory() as d:
        with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
            paths = list(ex.map(lambda s: _assembly(s, d), SOURCES))
        kernels = []
        for p in paths:
            kernels += _split_kernels(p)
        yield kernels


def test_no_mfma_result_used_early_after_a_taken_branch(assembly):
    straight, branched = {}, []
    for name, ins, labels in assembly:
        for op, dist, taken in _distances(ins, labels):
            if taken:
                branched.append((name, op, dist))
            else:
                straight[op] = min(straight.get(op, WINDOW), dist)
    assert straight, "no MFMA instruction found in the compiled kernels"
    bad = [(n, op, d, straight[op]) for n, op, d in branched if op in straight and d < straight[op]]
    assert not bad, "MFMA results used too early after a taken branch (kernel, opcode, distance, " \
                    "straight-line minimum): %s" % sorted(set(bad))[:10]


def _scan(lines):
    """Straight-line minimum and branched distances of a hand-written instruction list."""
    ins, labels = [], {}
    for line in lines:
        if line.endswith(":"):
            labels[line[:-1]] = len(ins)
            continue
        op = line.split()[0]
        ins.append((op, [o.strip() for o in line[len(op):].split(",")] if len(line) > len(op) else []))
    return _distances(ins, labels)


def test_scanner_rules_on_written_cases():
    mfma = "v_mfma_f32_16x16x16_bf16 v[0:3], v[4:5], v[6:7], v[0:3]"
    # straight line: a use four instructions after the MFMA
    assert _scan([mfma, "v_mov_b32 v8, v9", "v_mov_b32 v8, v9", "s_nop 1", "v_add_f32 v10, v0, v1"]) == \
        [("v_mfma_f32_16x16x16_bf16", 4, False)]
    # a taken branch to a use: found through the branch, at its distance
    found = _scan([mfma, "s_cbranch_scc1 .L1", "s_nop 7", "v_add_f32 v10, v0, v1", ".L1:", "v_add_f32 v11, v2, v3"])
    assert ("v_mfma_f32_16x16x16_bf16", 1, True) in found
    # exec known zero (execz taken): VALU instructions run on no lanes and are not uses ...
    found = _scan([mfma, "s_cbranch_execz .L1", "s_nop 7", "v_add_f32 v10, v0, v1", ".L1:",
                   "v_mov_b32 v2, v9", "s_endpgm"])
    assert all(not taken for _, _, taken in found)
    # ... but instructions that ignore exec are, and so is any VALU use once exec is written again
    found = _scan([mfma, "s_cbranch_execz .L1", "s_nop 7", "v_add_f32 v10, v0, v1", ".L1:",
                   "v_readlane_b32 s4, v1, 0", "s_endpgm"])
    assert ("v_mfma_f32_16x16x16_bf16", 1, True) in found
    found = _scan([mfma, "s_cbranch_execz .L1", "s_nop 7", "v_add_f32 v10, v0, v1", ".L1:",
                   "s_or_b64 exec, exec, s[6:7]", "v_mov_b32 v2, v9", "s_endpgm"])
    assert ("v_mfma_f32_16x16x16_bf16", 2, True) in found
    # falling through an execnz branch leaves exec zero as well: only the taken path's use counts
    found = _scan([mfma, "s_cbranch_execnz .L1", "v_mov_b32 v2, v9", "s_endpgm", ".L1:", "s_nop 7",
                   "v_mov_b32 v2, v9"])
    assert found == [("v_mfma_f32_16x16x16_bf16", 9, True)]
