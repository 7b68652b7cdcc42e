"""MFMA dependency rules around inline assembly in the 64-rows-per-wave kernel (csrc/attn_wide.h).

The compiler's hazard pass inserts the wait states between an MFMA and the instructions that depend on it,
but only for instructions it understands: an MFMA written as inline assembly, or an accumulator access inside
assembly, is invisible to it.  This test compiles the kernel to gfx950 assembly and scans it:
  - for an MFMA inside an assembly region: no VALU instruction may write one of its source registers within
    the 4 wait states before it, and no VALU instruction may read or write its destination within the 18
    wait states after it;
  - for a VALU instruction inside an assembly region (the accumulator rescale): no MFMA may have written a
    register it touches within the 18 wait states before it, unless a VALU instruction wrote that register
    again in between (the compiler makes its own writes wait for the MFMA).
A wait state is one instruction, or N+1 for s_nop N (an intervening MFMA counts as one, as in the hazard
rules).  18 covers the longest result latency of a 32x32 MFMA; 4 covers a VALU write read by an MFMA.
"""
from __future__ import annotations

import os
import re
import subprocess
import tempfile

import pytest

from dnn_compiler_pipelining_amd import build

KERNEL_SRCS = build.WIDE_SOURCES  # attn_wide.h, one placement per source
AFTER_MFMA = 18
BEFORE_MFMA = 4


def _regs(tok: str) -> set:
    tok = tok.strip()
    m = re.match(r"^-?\|?([va])\[(\d+):(\d+)\]\|?$", tok)
    if m:
        return {(m.group(1), i) for i in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.match(r"^-?\|?([va])(\d+)\|?$", tok)
    if m:
        return {(m.group(1), int(m.group(2)))}
    return set()


def _parse(line: str):
    parts = line.split(None, 1)
    ops = [x.strip() for x in parts[1].split(",")] if len(parts) > 1 else []
    return parts[0], ops


def _wait_states(op: str, ops) -> int:
    return int(ops[0]) + 1 if op == "s_nop" and ops else 1


def instructions(text: str, symbol: str):
    """[(in_asm, line)] of one kernel's body: in_asm marks instructions between ;;#ASMSTART and ;;#ASMEND."""
    start = text.index("\n" + symbol + ":")
    end = text.index(".Lfunc_end", start)
    out, in_asm = [], False
    for line in text[start:end].split("\n")[1:]:
        s = line.strip()
        if s.startswith(";;#ASMSTART"):
            in_asm = True
            continue
        if s.startswith(";;#ASMEND"):
            in_asm = False
            continue
        s = s.split(";")[0].strip()
        if not s or s.startswith(".") or s.endswith(":"):
            continue
        out.append((in_asm, s))
    return out


def scan(ins) -> list[str]:
    """The hazards described in the module docstring, as readable strings."""
    bad = []
    for i, (in_asm, line) in enumerate(ins):
        op, ops = _parse(line)
        if op.startswith("v_mfma") and in_asm:
            srcs = set().union(*[_regs(x) for x in ops[1:]]) if len(ops) > 1 else set()
            ws = 0
            for j in range(i - 1, -1, -1):
                op2, ops2 = _parse(ins[j][1])
                if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2 and _regs(ops2[0]) & srcs:
                    bad.append("VALU write %d wait states before an assembly MFMA: %s || %s" % (ws, ins[j][1], line))
                ws += _wait_states(op2, ops2)
                if ws >= BEFORE_MFMA:
                    break
            dst = _regs(ops[0])
            ws = 0
            for j in range(i + 1, len(ins)):
                op2, ops2 = _parse(ins[j][1])
                if op2.startswith("v_") and not op2.startswith("v_mfma") and ops2 and \
                        set().union(*[_regs(x) for x in ops2]) & dst:
                    bad.append("VALU access %d wait states after an assembly MFMA: %s || %s" % (ws, line, ins[j][1]))
                ws += _wait_states(op2, ops2)
                if ws >= AFTER_MFMA:
                    break
        elif in_asm and op.startswith("v_") and not op.startswith("v_mfma"):
            # registers whose latest writer could still be an MFMA: a later VALU write of a register hides an
            # earlier MFMA write of it (the later writer is the one that has to wait for the MFMA)
            touched = set().union(*[_regs(x) for x in ops]) if ops else set()
            ws = 0
            for j in range(i - 1, -1, -1):
                op2, ops2 = _parse(ins[j][1])
                ws += _wait_states(op2, ops2) if j < i - 1 else 0
                if op2.startswith("v_mfma") and ops2 and _regs(ops2[0]) & touched:
                    bad.append("assembly VALU access %d wait states after an MFMA: %s || %s" % (ws, ins[j][1], line))
                elif op2.startswith("v_") and ops2:
                    touched -= _regs(ops2[0])
                if ws >= AFTER_MFMA or not touched:
                    break
    return bad


def test_scanner_finds_planted_hazards():
    """The scanner itself, on hand-written sequences: each planted hazard is found, the safe forms are not."""
    mfma_asm = (True, "v_mfma_f32_32x32x16_f16 v[0:15], v[16:19], a[0:3], v[0:15]")
    # a VALU write of a source right before an assembly MFMA
    assert scan([(False, "v_mov_b32_e32 v17, 0"), mfma_asm])
    # a VALU read of the result right after
    assert scan([mfma_asm, (False, "v_add_f32_e32 v30, v3, v3")])
    # an assembly accumulator read right after a builtin MFMA that wrote it
    assert scan([(False, "v_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]"),
                 (True, "v_accvgpr_read_b32 v40, a5")])
    # an assembly accumulator read of a register the VALU rewrote after the MFMA wrote it: clean
    assert not scan([(False, "v_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]"),
                     (False, "v_accvgpr_mov_b32 a5, a40"),
                     (True, "v_accvgpr_read_b32 v40, a5")])
    # ... but a register the rewrite does not cover still counts
    assert scan([(False, "v_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]"),
                 (False, "v_accvgpr_mov_b32 a5, a40"),
                 (True, "v_accvgpr_read_b32 v40, a6")])
    # the same with enough wait states between, and with unrelated registers: clean
    assert not scan([mfma_asm, (True, "s_nop 7"), (True, "s_nop 7"), (True, "s_nop 2"),
                     (False, "v_add_f32_e32 v30, v3, v3")])
    assert not scan([(False, "v_mov_b32_e32 v40, 0"), mfma_asm, (False, "v_add_f32_e32 v41, v40, v40")])
    assert not scan([(False, "v_mfma_f32_32x32x16_f16 a[0:15], v[0:3], v[4:7], a[0:15]"),
                     (True, "v_accvgpr_read_b32 v40, a20")])


@pytest.fixture(scope="module")
def wide_asm():
    paths = []
    for _ in KERNEL_SRCS:
        fd, path = tempfile.mkstemp(suffix=".s")
        os.close(fd)
        paths.append(path)
    try:
        build.device_asm_many(zip(paths, KERNEL_SRCS))
        texts = []
        for path in paths:
            with open(path) as f:
                texts.append(f.read())
        yield texts
    finally:
        for path in paths:
            os.remove(path)


def test_wide_kernel_keeps_the_mfma_dependency_rules(wide_asm):
    n = 0
    for text in wide_asm:
        symbols = re.findall(r"^(_ZN7libattn16attn_wide_kernel\S*):", text, re.M)
        assert symbols, "no wide kernel in the assembly"
        for sym in symbols:
            ins = instructions(text, sym)
            assert sum(1 for a, l in ins if a and l.startswith("v_mfma")) >= 32, sym
            bad = scan(ins)
            assert not bad, "%s:\n%s" % (sym, "\n".join(bad[:20]))
            n += 1
    assert n == 6  # two prefetch depths x three placements
