"""Static check of AMD GPU assembly for one MFMA hazard seen on gfx950.

On this part (ROCm 7.2 compiler) a bf16 MFMA whose accumulator input (SrcC) is
the result of the other bf16 MFMA shape, issued back to back, reads stale
values in half of its accumulator rows: tests/hip/mfma_chain.hip shows
16x16x32 -> 16x16x16 with the 2 wait states the compiler inserts wrong in rows
4g and 4g + 1 of every 16-row tile, 16x16x16 -> 16x16x32 with none wrong in rows
4g + 2 and 4g + 3, and both right with 16 more wait states.  This module finds
such chains in compiled assembly: an MFMA reading SrcC from registers last
written by an MFMA of a different opcode fewer than MIN_WAIT wait states earlier
(s_nop N counts N + 1, any other instruction 1), scanning each function's
instructions in order (a chain across a loop's back edge is not seen).
"""
from __future__ import annotations

import re

MIN_WAIT = 16
_REG = re.compile(r"^([av])\[(\d+):(\d+)\]$|^([av])(\d+)$")


def _regs(tok: str):
    m = _REG.match(tok.strip())
    if not m:
        return None
    if m.group(1):
        return (m.group(1), int(m.group(2)), int(m.group(3)))
    return (m.group(4), int(m.group(5)), int(m.group(5)))


def _overlap(a, b):
    return a[0] == b[0] and a[1] <= b[2] and b[1] <= a[2]


def find_chains(asm: str):
    """[(function, line, first opcode, second opcode, wait states)] of every
    MFMA whose SrcC comes from a different MFMA opcode too few wait states back."""
    found = []
    func = None
    recent = []  # (vdst regs, opcode, wait states since)
    for lineno, raw in enumerate(asm.splitlines(), 1):
        line = raw.split(";")[0].strip()
        if not line:
            continue
        if line.endswith(":") and not line.startswith("."):
            if not line.startswith(".L"):
                func = line[:-1]
                recent = []
            continue
        if line.startswith("."):
            continue
        parts = line.split(None, 1)
        op = parts[0]
        args = [a.strip() for a in parts[1].split(",")] if len(parts) > 1 else []
        cost = int(args[0], 0) + 1 if op == "s_nop" and args else 1
        if op.startswith("v_mfma") and len(args) >= 4:
            src_c = _regs(args[3])
            if src_c is not None:
                for dst, prev_op, since in recent:
                    if _overlap(dst, src_c) and prev_op != op and since < MIN_WAIT:
                        found.append((func, lineno, prev_op, op, since))
                        break
            dst = _regs(args[0])
            # the new write supersedes older entries on the same registers
            recent = [(d, o, s + cost) for d, o, s in recent
                      if dst is None or not _overlap(d, dst)]
            if dst is not None:
                recent.append((dst, op, 0))
            continue
        recent = [(d, o, s + cost) for d, o, s in recent if s + cost < 4 * MIN_WAIT]
    return found
