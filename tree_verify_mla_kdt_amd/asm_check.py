"""Build-time check of the split kernel's inline-asm score MFMAs.

The score contraction's MFMAs are written as inline asm (so that the tile
they accumulate stays in ordinary VGPRs), and the compiler's hazard
recognizer does not look inside inline asm.  The one hazard those
instructions can meet from the code around them is a vector ALU instruction
writing an A or B operand register fewer than two wait states before the
MFMA reads it (the accumulation itself runs back to back into the same
registers, which the hardware allows, and the kernel separates the last
MFMA from the first vector read of the tile with explicit wait states).  This
module scans the compiled assembly of every kernel for that pattern, and for
an MFMA destination overlapping its A or B operand, following branches back
into predecessor blocks, and the build fails if it finds one.
"""
from __future__ import annotations

import re

_MFMA = re.compile(r"v_mfma_\w+\s+(v\[\d+:\d+\]|v\d+),\s*(v\[\d+:\d+\]|v\d+),\s*(v\[\d+:\d+\]|v\d+)")
_LABEL = re.compile(r"^(\.LBB\w+|\.L\w+):")
_BRANCH = re.compile(r"^s_(?:c?branch\w*)\s+(\.L\w+)")
_NOP = re.compile(r"^s_nop\s+(\d+)")
NEED = 2          # wait states between a vector ALU write and an MFMA read of the register


def _regs(tok: str) -> set[int]:
    m = re.match(r"v\[(\d+):(\d+)\]$", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def _valu_dst(ins: str) -> set[int]:
    """VGPRs written by a vector ALU instruction (not an MFMA), else empty."""
    if not ins.startswith("v_") or ins.startswith("v_mfma") or ins.startswith(("v_readlane", "v_readfirstlane",
                                                                             "v_cmp")):
        return set()
    parts = ins.split(None, 1)
    if len(parts) < 2:
        return set()
    return _regs(parts[1].split(",")[0].strip())


def _functions(asm: str):
    for m in re.finditer(r"^(\w+):\s*(?:;.*)?$", asm, re.M):
        name = m.group(1)
        end = asm.find(".Lfunc_end", m.end())
        if end < 0 or not name.startswith("_Z"):
            continue
        yield name, asm[m.end():end]


def check(asm: str) -> list[str]:
    problems = []
    for name, text in _functions(asm):
        lines = []
        for raw in text.split("\n"):
            x = raw.split(";")[0].strip()
            if x and not (x.startswith(".") and not _LABEL.match(x)):
                lines.append(x)
        labels = {}
        branches: dict[str, list[int]] = {}
        for i, x in enumerate(lines):
            m = _LABEL.match(x)
            if m:
                labels[m.group(1)] = i
            m = _BRANCH.match(x)
            if m:
                branches.setdefault(m.group(1), []).append(i)

        def look_back(i: int, budget: int, src: set[int], seen: set) -> str | None:
            """Walk back from line i (exclusive) over `budget` wait states."""
            while budget > 0:
                i -= 1
                if i < 0:
                    return None
                x = lines[i]
                m = _LABEL.match(x)
                if m:
                    for b in branches.get(m.group(1), []):
                        key = (b, budget)
                        if key not in seen:
                            seen.add(key)
                            # the branch itself is one wait state
                            r = look_back(b, budget - 1, src, seen)
                            if r:
                                return r
                    continue
                if x.startswith("s_branch"):
                    return None            # not a fall-through predecessor
                n = _NOP.match(x)
                if n:
                    budget -= int(n.group(1)) + 1
                    continue
                if _valu_dst(x) & src:
                    return x
                budget -= 1
            return None

        for i, x in enumerate(lines):
            m = _MFMA.match(x)
            if not m:
                continue
            dst, a, b = (_regs(t) for t in m.groups())
            src = a | b
            if dst & src and dst:
                problems.append(f"{name}: destination overlaps an operand: {x}")
            w = look_back(i, NEED, src, set())
            if w:
                problems.append(f"{name}: '{w}' writes an operand of '{x}' too soon")
    return problems
